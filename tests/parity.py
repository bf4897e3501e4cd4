"""Shared helpers for the GPU parity tests: moving the seeded inputs to the
device, running libmdn and the oracle on the same values, and the tolerance
rules.

Tolerances (written here once, used by every parity test):
  fp32 I/O: for each result tensor X with oracle X*,
            max|X - X*| / max|X*| <= 1e-4     (relative to the tensor's scale;
            elementwise relative error is ill-posed where X* crosses 0)
  bf16 I/O: max|X - X*| <= 2e-2 * max(1, rms(X*)) per tensor; the outputs are
            unit scale, so this is an absolute 2e-2 bound.  Beside it, a
            companion bound relative to the tensor's own scale:
            max|X - X*| <= 2e-2 * max|X*|.  The final states (and the decode
            state and early decode outputs) are far below unit scale (M_T has
            an rms of a few 1e-2), where the absolute bound alone would let an
            error of the size of the signal pass.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from chunkwise_delta_rule_amd import mdn

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
FP32_REL_TOL = 1e-4
BF16_ABS_TOL = 2e-2
BF16_REL_TOL = 2e-2


def to_dev(x, dtype=torch.float32):
    if x is None:
        return None
    # float32 holding values exactly representable in `dtype`: exact cast
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype)


def to_np(t):
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_forward(inp, mu=None, S0=None, M0=None, io=None, beta="inp", mu_null=False):
    """beta: "inp" passes the workload's own beta (None if it has none), or
    give an array or None explicitly.  mu_null passes no mu (mu = 0)."""
    io = io or inp["cfg"].io_dtype
    dt = TORCH_DT[io]
    beta = inp.get("beta") if isinstance(beta, str) else beta
    mu_dev = None if mu_null else to_dev(inp["mu"] if mu is None else mu)
    O, ST, MT = mdn.chunk_fwd(to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
                              to_dev(inp["alpha"]), mu_dev,
                              to_dev(inp["eta"]),
                              to_dev(inp["S0"] if S0 is None else S0),
                              to_dev(inp["M0"] if M0 is None else M0), beta=to_dev(beta))
    torch.cuda.synchronize()
    return to_np(O), to_np(ST), to_np(MT)


def split_forward(inp, io=None, mu_null=False):
    """The same forward through the two exported phases (prepare, then scan)."""
    io = io or inp["cfg"].io_dtype
    dt = TORCH_DT[io]
    plan = mdn.ChunkPlan(to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
                         to_dev(inp["alpha"]), None if mu_null else to_dev(inp["mu"]),
                         to_dev(inp["eta"]),
                         to_dev(inp["S0"]), to_dev(inp["M0"]), beta=to_dev(inp.get("beta")))
    plan.O.fill_(float("nan"))
    plan.S_T.fill_(float("nan"))
    plan.M_T.fill_(float("nan"))
    plan.prepare()
    plan.scan()
    torch.cuda.synchronize()
    return to_np(plan.O), to_np(plan.S_T), to_np(plan.M_T)


def gather_heads(x, pairs, state=False):
    """Stack the (b, h) pairs of a [B, T, H, ...] (or [B, H, ...] state)
    array along a new head axis of a batch of one."""
    if x is None:
        return None
    if state:
        return np.stack([x[b, h] for b, h in pairs], axis=0)[None]
    return np.stack([x[b, :, h] for b, h in pairs], axis=1)[None]


def oracle_forward(inp, pairs=None, mu=None):
    mu = inp["mu"] if mu is None else mu
    beta = inp.get("beta")
    if pairs is None:
        return oracle.recurrence(inp["q"], inp["k"], inp["v"], inp["alpha"], mu, inp["eta"], beta,
                                 inp["S0"], inp["M0"])
    g = lambda x: gather_heads(x, pairs)
    return oracle.recurrence(g(inp["q"]), g(inp["k"]), g(inp["v"]), g(inp["alpha"]), g(mu),
                             g(inp["eta"]), g(beta), gather_heads(inp["S0"], pairs, True),
                             gather_heads(inp["M0"], pairs, True))


def errors(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    err = float(np.max(np.abs(x - ref))) if x.size else 0.0
    mx = float(np.max(np.abs(ref))) if ref.size else 0.0
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return err, mx, rms


def assert_close(x, ref, io, name):
    assert x.shape == ref.shape, (name, x.shape, ref.shape)
    assert np.all(np.isfinite(x)), f"{name}: non-finite values"
    err, mx, rms = errors(x, ref)
    if io == "f32":
        rel = err / mx if mx > 0 else err
        print(f"  {name}: max|err|={err:.3e} max|ref|={mx:.3e} rel={rel:.3e} (tol {FP32_REL_TOL})")
        assert rel <= FP32_REL_TOL, f"{name}: relative error {rel:.3e} > {FP32_REL_TOL}"
    else:
        bound = BF16_ABS_TOL * max(1.0, rms)
        rel = err / mx if mx > 0 else err
        print(f"  {name}: max|err|={err:.3e} bound={bound:.3e} rel={rel:.3e} "
              f"(tol {BF16_REL_TOL}) max|ref|={mx:.3e} rms={rms:.3e}")
        assert err <= bound, f"{name}: max abs error {err:.3e} > {bound:.3e}"
        assert rel <= BF16_REL_TOL, f"{name}: error {rel:.3e} of max|ref| > {BF16_REL_TOL}"
