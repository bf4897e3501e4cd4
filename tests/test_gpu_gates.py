"""GPU parity of mdn_gates_from_logits (MDN's coupled gates, "MDN:
Parallelizing Stepwise Momentum for Delta Linear Attention" (slides), frame
"Coupled gates restrict the spectral region") against the oracle's float64
gates_from_logits, element by element, through the C ABI.

Tolerance, per element with oracle value r and kernel value x:
    |x - r| <= 8 * 2^-24 * (2 + |ln r|) * r + atol
Each gate is an exponential (or a ratio of them) of an argument the kernel
forms in float32 from float32 logits and parameters: the argument carries a
few half-ulps of relative error, which the exponential turns into a relative
error of about |argument| = |ln r| half-ulps, plus a few ulps of the final
rounding.  atol covers values below float32's normal range (1e-37, alpha and
mu) and the float64 rounding of the literal 1 + tanh that the oracle
evaluates for eta (1e-15, eta and beta).  The oracle is called with the
float32-rounded parameters the kernel receives.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from chunkwise_delta_rule_amd import mdn

pytestmark = pytest.mark.gpu

EPS32 = 2.0 ** -24
ATOL = {"alpha": 1e-37, "mu": 1e-37, "eta": 1e-15, "beta": 1e-15}
# (tau, s, a, b, log_mu_min): the pages' floor -2 and the text's -1, a
# temperature sqrt(d_in / h) for d_in = 2048, h = 16, and a weak decay scale
PARAMS = [
    (2.5, 1.7, 0.8, 0.3, -2.0),
    (11.3137, 0.5, 1.0, -1.0, -1.0),
    (1.0, 3.0, 0.05, 2.0, -2.0),
]


def f32(x):
    return float(np.float32(x))


def run_gpu(z, params, shape=None):
    dev = lambda x: torch.from_numpy(x).to("cuda").reshape(shape or x.shape)
    tau, s, a, b, fl = params
    out = mdn.gates_from_logits(dev(z["z_eta"]), dev(z["z_alpha"]), dev(z["z_beta"]),
                                dev(z["z_mu"]), tau=tau, s=s, a=a, b=b, log_mu_min=fl)
    torch.cuda.synchronize()
    return [t.cpu().numpy().reshape(-1).astype(np.float64) for t in out]


def run_oracle(z, params):
    tau, s, a, b, fl = (f32(p) for p in params)
    return oracle.gates_from_logits(z["z_eta"], z["z_alpha"], z["z_beta"], z["z_mu"], tau=tau,
                                    s=s, a=a, b=b, log_mu_min=fl)


def assert_gates_close(got, ref, label):
    for name, x, r in zip(("alpha", "mu", "eta", "beta"), got, ref):
        assert x.shape == r.shape, (name, x.shape, r.shape)
        assert np.all(np.isfinite(x)), f"{label} {name}: non-finite values"
        with np.errstate(divide="ignore"):
            lnr = np.where(r > 0, np.abs(np.log(np.where(r > 0, r, 1.0))), 0.0)
        tol = 8 * EPS32 * (2.0 + lnr) * np.abs(r) + ATOL[name]
        ratio = np.abs(x - r) / tol
        i = int(np.argmax(ratio)) if ratio.size else 0
        worst = float(ratio[i]) if ratio.size else 0.0
        print(f"  {label} {name}: max err/tol = {worst:.3f}")
        assert worst <= 1.0, (f"{label} {name}[{i}]: got {x[i]!r}, oracle {r[i]!r}, "
                              f"err/tol {worst:.3f}")


@pytest.mark.parametrize("n", [1, 3, 4, 7, 64, 1000, 4099, 8 * 4096 * 16 + 3])
@pytest.mark.parametrize("pi", range(len(PARAMS)))
def test_gates_match_oracle(n, pi):
    z = si.gate_logits(n, seed=100 + pi)
    print(f"gates n={n} params={PARAMS[pi]}", flush=True)
    assert_gates_close(run_gpu(z, PARAMS[pi]), run_oracle(z, PARAMS[pi]), f"n={n}")


def test_gates_grid_stride_beyond_one_sweep():
    # the launch caps the grid at 16384 workgroups of 256 threads, 2 values
    # each: 2^23 values per sweep; this covers two sweeps and a ragged tail
    n = 2 * (16384 * 256 * 2) + 1001
    z = si.gate_logits(n, seed=7)
    print(f"gates n={n}", flush=True)
    assert_gates_close(run_gpu(z, PARAMS[0]), run_oracle(z, PARAMS[0]), f"n={n}")


def test_gates_shared_input_buffer():
    # the four logits may be one buffer: all gates from the same values
    n = 1000
    z1 = si.gate_logits(n, seed=11)["z_alpha"]
    t = torch.from_numpy(z1).to("cuda")
    out = mdn.gates_from_logits(t, t, t, t, tau=2.0, s=1.0, a=1.0, b=0.0, log_mu_min=-2.0)
    torch.cuda.synchronize()
    got = [g.cpu().numpy().astype(np.float64) for g in out]
    z = dict(z_eta=z1, z_alpha=z1, z_beta=z1, z_mu=z1)
    assert_gates_close(got, run_oracle(z, (2.0, 1.0, 1.0, 0.0, -2.0)), "shared")


def test_gates_zero_length_is_a_no_op():
    e = torch.empty(0, device="cuda")
    out = mdn.gates_from_logits(e, e, e, e, tau=1.0, s=1.0, a=1.0, b=0.0)
    torch.cuda.synchronize()
    assert all(g.numel() == 0 for g in out)


def test_gates_feed_the_forward():
    """Logits -> gates -> chunkwise forward on the GPU against the oracle's
    gates -> the oracle's recurrence (fp32, a ragged T over several chunks)."""
    from parity import assert_close, to_dev, to_np

    cfg = si.ForwardConfig(name="gates", B=1, T=200, H=3, Dk=64, Dv=64, chunk=64,
                           io_dtype="f32", gates="uniform", seed=41)
    inp = si.make_forward(cfg)
    z = si.gate_logits(cfg.B * cfg.T * cfg.H, seed=42, scale=2.0)
    params = (2.0, 1.0, 0.5, 1.0, -2.0)
    shape = (cfg.B, cfg.T, cfg.H)
    dev = lambda x: torch.from_numpy(x).to("cuda").reshape(shape)
    alpha, mu, eta, beta = mdn.gates_from_logits(
        dev(z["z_eta"]), dev(z["z_alpha"]), dev(z["z_beta"]), dev(z["z_mu"]),
        tau=params[0], s=params[1], a=params[2], b=params[3], log_mu_min=params[4])
    O, ST, MT = mdn.chunk_fwd(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), alpha, mu,
                              eta, None, None, beta=beta)
    torch.cuda.synchronize()
    ra, rm, re, rb = (g.reshape(shape) for g in run_oracle(z, params))
    ref = oracle.recurrence(inp["q"], inp["k"], inp["v"], ra, rm, re, rb, None, None)
    for name, x, r in zip(("O", "S_T", "M_T"), (to_np(O), to_np(ST), to_np(MT)), ref):
        assert_close(x, r, "f32", name)
