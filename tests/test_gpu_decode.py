"""GPU parity of mdn_decode_step against the fp64 oracle, through the C ABI.

The decode loop of 256 sequences x 16 heads (d = 128) runs all 512 steps on
the GPU with fresh seeded tokens each step; the oracle follows every
(sequence, head) pair through every step, and o is compared at every step
for all of them, then the final S and M.  Small shapes cover every head-size pair
and both I/O dtypes.  Tolerances are in parity.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from chunkwise_delta_rule_amd import mdn
from parity import BF16_ABS_TOL, BF16_REL_TOL, TORCH_DT, assert_close, errors, to_dev, to_np

pytestmark = pytest.mark.gpu


def run_decode(cfg, pairs=None, steps=None):
    """Run `steps` decode steps on the GPU and the oracle (on `pairs` or all
    heads).  Returns the worst per-step o error and the final states."""
    steps = cfg.steps if steps is None else steps
    dt = TORCH_DT[cfg.io_dtype]
    stream = si.decode_stream(cfg)
    S0, M0 = next(stream)
    S = to_dev(S0)
    M = to_dev(M0)
    if pairs is None:
        pairs = [(n, h) for n in range(cfg.N) for h in range(cfg.H)]
    ni = np.array([p[0] for p in pairs])
    hi = np.array([p[1] for p in pairs])
    Sr = S0[ni, hi][:, None].astype(np.float64)          # [P, 1, Dk, Dv]
    Mr = M0[ni, hi][:, None].astype(np.float64)
    worst = (0.0, 0.0, 0.0)
    for step in range(steps):
        tok = next(stream)
        beta = tok.get("beta")
        o = mdn.decode_step(to_dev(tok["q"], dt), to_dev(tok["k"], dt), to_dev(tok["v"], dt),
                            to_dev(tok["alpha"]), to_dev(tok["mu"]), to_dev(tok["eta"]), S, M,
                            beta=to_dev(beta))
        sel = lambda x: None if x is None else x[ni, hi][:, None]
        o_ref, Sr, Mr = oracle.decode_step(sel(tok["q"]), sel(tok["k"]), sel(tok["v"]),
                                           sel(tok["alpha"]), sel(tok["mu"]), sel(tok["eta"]),
                                           Sr, Mr, sel(beta))
        o_got = to_np(o)[ni, hi][:, None]
        err = errors(o_got, o_ref)
        if err[0] > worst[0]:
            worst = err
        if cfg.io_dtype == "f32":
            assert_close(o_got, o_ref, "f32", f"o step {step}")
        elif err[0] > BF16_ABS_TOL * max(1.0, err[2]) or err[0] > BF16_REL_TOL * err[1]:
            assert_close(o_got, o_ref, "bf16", f"o step {step}")
    torch.cuda.synchronize()
    Sg = to_np(S)[ni, hi][:, None]
    Mg = to_np(M)[ni, hi][:, None]
    return worst, (Sg, Mg), (Sr, Mr)


SMALL = [(io, dk, dv) for io in ("f32", "bf16") for (dk, dv) in
         ((64, 64), (64, 128), (128, 64), (128, 128))]


@pytest.mark.parametrize("io,dk,dv", SMALL, ids=[f"{a}-dk{b}-dv{c}" for a, b, c in SMALL])
def test_decode_small(io, dk, dv):
    cfg = dataclasses.replace(si.CONFIGS[4], N=3, H=5, Dk=dk, Dv=dv, steps=20, state_std=0.3,
                              io_dtype=io, seed=4000 + dk + dv)
    worst, got, ref = run_decode(cfg)
    print(f"[decode {io} dk{dk} dv{dv}] worst o err {worst[0]:.3e} (max|o| {worst[1]:.3e})")
    assert_close(got[0], ref[0], io, "S")
    assert_close(got[1], ref[1], io, "M")


@pytest.mark.parametrize("io,d", [("f32", 64), ("bf16", 128)])
def test_decode_beta_gate(io, d):
    """The four-gate form: a fresh update-step gate beta = sigmoid(z) each
    step, against the oracle's beta recurrence."""
    cfg = dataclasses.replace(si.CONFIGS[4], N=3, H=5, Dk=d, Dv=d, steps=20, state_std=0.3,
                              io_dtype=io, beta="logit", seed=4500 + d)
    worst, got, ref = run_decode(cfg)
    print(f"[decode beta {io} d{d}] worst o err {worst[0]:.3e} (max|o| {worst[1]:.3e})")
    assert_close(got[0], ref[0], io, "S")
    assert_close(got[1], ref[1], io, "M")


def test_decode_beta_ones_matches_no_beta_bitwise():
    """An all-ones beta runs exactly the arithmetic of no beta."""
    cfg = dataclasses.replace(si.CONFIGS[4], N=2, H=3, steps=1, state_std=0.3)
    stream = si.decode_stream(cfg)
    S0, M0 = next(stream)
    tok = next(stream)
    dt = torch.bfloat16
    outs = []
    for beta in (None, np.ones_like(tok["alpha"])):
        S, M = to_dev(S0), to_dev(M0)
        o = mdn.decode_step(to_dev(tok["q"], dt), to_dev(tok["k"], dt), to_dev(tok["v"], dt),
                            to_dev(tok["alpha"]), to_dev(tok["mu"]), to_dev(tok["eta"]), S, M,
                            beta=to_dev(beta))
        torch.cuda.synchronize()
        outs.append((to_np(o), to_np(S), to_np(M)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("keep_m", [False, True])
def test_decode_mu_null(keep_m):
    """No mu (mu = 0): the momentum-free step over 20 tokens against the
    oracle at mu = 0; without M only S is kept, with M it receives each
    step's own write."""
    cfg = dataclasses.replace(si.CONFIGS[4], N=3, H=5, steps=20, state_std=0.3, seed=4600)
    stream = si.decode_stream(cfg)
    S0, M0 = next(stream)
    S = to_dev(S0)
    M = to_dev(M0) if keep_m else None
    Sr = S0.reshape(cfg.N * cfg.H, 1, cfg.Dk, cfg.Dv).astype(np.float64)
    Mr = M0.reshape(cfg.N * cfg.H, 1, cfg.Dk, cfg.Dv).astype(np.float64)
    dt = torch.bfloat16
    flat = lambda x: x.reshape(cfg.N * cfg.H, 1, *x.shape[2:])
    for step in range(cfg.steps):
        tok = next(stream)
        o = mdn.decode_step(to_dev(tok["q"], dt), to_dev(tok["k"], dt), to_dev(tok["v"], dt),
                            to_dev(tok["alpha"]), None, to_dev(tok["eta"]), S, M)
        zero = np.zeros((cfg.N * cfg.H, 1), np.float32)
        o_ref, Sr, Mr = oracle.decode_step(flat(tok["q"]), flat(tok["k"]), flat(tok["v"]),
                                           tok["alpha"].reshape(-1, 1), zero,
                                           tok["eta"].reshape(-1, 1), Sr, Mr)
        assert_close(to_np(o).reshape(o_ref.shape), o_ref, "bf16", f"o step {step}")
    torch.cuda.synchronize()
    assert_close(to_np(S).reshape(Sr.shape), Sr, "bf16", "S")
    if keep_m:
        assert_close(to_np(M).reshape(Mr.shape), Mr, "bf16", "M")


def run_decode_all_heads(cfg, block=32):
    """Every (sequence, head) through every step.  The GPU runs the decode
    steps one by one, keeping every step's o; the oracle runs the same tokens
    as one recurrence over the chain of steps (a decode step is the
    recurrence at T = 1, so a chain of them is the recurrence over the
    chain), `block` sequences at a time.  o is checked step by step over all
    heads, then the final S and M."""
    dt = TORCH_DT[cfg.io_dtype]
    stream = si.decode_stream(cfg)
    S0, M0 = next(stream)
    S, M = to_dev(S0), to_dev(M0)
    O = torch.empty((cfg.steps, cfg.N, cfg.H, cfg.Dv), dtype=dt, device="cuda")
    toks = []
    for step in range(cfg.steps):
        tok = next(stream)
        toks.append(tok)
        mdn.decode_step(to_dev(tok["q"], dt), to_dev(tok["k"], dt), to_dev(tok["v"], dt),
                        to_dev(tok["alpha"]), to_dev(tok["mu"]), to_dev(tok["eta"]), S, M,
                        o=O[step], beta=to_dev(tok.get("beta")))
    torch.cuda.synchronize()
    print(f"decode: {cfg.steps} GPU steps done; oracle", flush=True)
    Og = O.float().cpu().numpy()                      # [steps, N, H, Dv]
    Sg, Mg = to_np(S), to_np(M)
    del O, S, M
    # per step: max error, max |o*| and sum of o*^2 over all heads
    err = np.zeros(cfg.steps)
    mx = np.zeros(cfg.steps)
    ss = np.zeros(cfg.steps)
    Sr = np.zeros_like(Sg)
    Mr = np.zeros_like(Mg)
    has_beta = toks[0].get("beta") is not None
    for n0 in range(0, cfg.N, block):
        sl = slice(n0, min(cfg.N, n0 + block))
        seq = lambda name: np.stack([t[name][sl] for t in toks], axis=1)
        O_ref, Sr[sl], Mr[sl] = oracle.recurrence(
            seq("q"), seq("k"), seq("v"), seq("alpha"), seq("mu"), seq("eta"),
            seq("beta") if has_beta else None, S0[sl], M0[sl])
        got = np.moveaxis(Og[:, sl], 0, 1)           # [nb, steps, H, Dv]
        assert np.all(np.isfinite(got))
        e = np.abs(got - O_ref).max(axis=(0, 2, 3))
        err = np.maximum(err, e)
        mx = np.maximum(mx, np.abs(O_ref).max(axis=(0, 2, 3)))
        ss += (O_ref * O_ref).sum(axis=(0, 2, 3))
    rms = np.sqrt(ss / (cfg.N * cfg.H * cfg.Dv))
    return err, mx, rms, (Sg, Mg), (Sr, Mr)


def test_decode_full_config_all_heads():
    """256 x 16 heads, d = 128, 512 steps (the benchmarked launch), every
    head and element: o at every step, then S and M."""
    cfg = si.CONFIGS[4]
    err, mx, rms, got, ref = run_decode_all_heads(cfg)
    abs_bound = BF16_ABS_TOL * np.maximum(1.0, rms)
    rel = err / mx
    w = int(np.argmax(err / abs_bound))
    wr = int(np.argmax(rel))
    print(f"[decode N256 H16 d128 x512, all heads] o: worst step {w}: max|err| {err[w]:.3e} "
          f"bound {abs_bound[w]:.3e}; worst relative step {wr}: {rel[wr]:.3e} of max|o*| "
          f"{mx[wr]:.3e} (tol {BF16_REL_TOL})")
    assert np.all(err <= abs_bound), np.nonzero(err > abs_bound)[0][:10]
    assert np.all(rel <= BF16_REL_TOL), np.nonzero(rel > BF16_REL_TOL)[0][:10]
    assert_close(got[0], ref[0], "bf16", "S")
    assert_close(got[1], ref[1], "bf16", "M")


def test_decode_matches_forward():
    """Decode steps chained over T tokens equal one chunkwise forward over the
    same tokens (outputs and final states), both against the oracle."""
    inp = si.make_forward(si.CONFIGS[1], B=2, T=150, H=3, init_state_std=0.2, seed=9)
    dt = torch.bfloat16
    S = to_dev(inp["S0"])
    M = to_dev(inp["M0"])
    outs = []
    for t in range(150):
        outs.append(mdn.decode_step(to_dev(inp["q"][:, t], dt), to_dev(inp["k"][:, t], dt),
                                    to_dev(inp["v"][:, t], dt), to_dev(inp["alpha"][:, t]),
                                    to_dev(inp["mu"][:, t]), to_dev(inp["eta"][:, t]), S, M))
    O_dec = to_np(torch.stack(outs, dim=1))
    O_fwd, S_fwd, M_fwd = mdn.chunk_fwd(to_dev(inp["q"], dt), to_dev(inp["k"], dt),
                                        to_dev(inp["v"], dt), to_dev(inp["alpha"]),
                                        to_dev(inp["mu"]), to_dev(inp["eta"]),
                                        to_dev(inp["S0"]), to_dev(inp["M0"]))
    torch.cuda.synchronize()
    ref = oracle.recurrence(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["mu"], inp["eta"],
                            None, inp["S0"], inp["M0"])
    print("[decode chain vs forward]")
    assert_close(O_dec, ref[0], "bf16", "O (decode)")
    assert_close(to_np(S), ref[1], "bf16", "S (decode)")
    assert_close(to_np(M), ref[2], "bf16", "M (decode)")
    assert_close(O_dec, to_np(O_fwd), "bf16", "O decode vs forward")
    assert_close(to_np(S), to_np(S_fwd), "bf16", "S decode vs forward")


def test_decode_bad_arguments_raise():
    dt = torch.bfloat16
    x = torch.zeros(2, 2, 64, dtype=dt, device="cuda")
    g = torch.zeros(2, 2, device="cuda")
    S = torch.zeros(2, 2, 64, 64, device="cuda")
    with pytest.raises(mdn.MdnError) as ex:
        mdn.decode_step(x, x, x, g, g, g, S, S)        # S and M are the same buffer
    assert ex.value.status == 5
