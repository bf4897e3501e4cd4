"""GPU parity of mdn_chunk_bwd (the backward pass through mdn_chunk_fwd)
against the oracle's reverse-mode derivative of the token recurrence
(oracle.recurrence_backward, itself pinned by finite differences), element
by element, on the same seeded inputs and output gradients.

Tolerance, per result tensor X with oracle X* (the whole tensor's scale:
elementwise relative error is ill-posed where X* crosses 0):
  fp32 I/O:  max|X - X*| <= 2e-5 max|X*|
  bf16 I/O:  max|X - X*| <= 1e-2 max|X*|
For fp32 I/O the backward computes in fp32 (measured: under 1e-6 of the
scale on the small cases).  For bf16 I/O its products run on bf16 MFMA with
fp32 sums: the inputs, T = L^-1 and A (stored in bf16 by the prepare phase)
and the saved residuals are exact as operands; the per-chunk state pairs the
backward keeps are stored in bf16, and its fp32 row operands are split into a
bf16 head and remainder or rounded once.  That moves every gradient by a few
1e-3 of its scale (measured up to about 9e-3 with saved residuals on a
65-token case); the full-size cases print their worst ratio to the bound.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from chunkwise_delta_rule_amd import mdn
from parity import TORCH_DT, gather_heads, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-5, "bf16": 1e-2}
NAMES = ("dq", "dk", "dv", "dalpha", "dmu", "deta", "dbeta", "dS0", "dM0")


def run_case(cfg, *, seed=5, terminal=True, mu_null=False, with_beta=False, label="",
             heads=None, saved=False):
    """heads: (b, h) pairs to compare (all when None); the GPU always runs the
    whole workload."""
    inp = si.make_forward(cfg)
    cot = si.backward_cotangents(cfg, seed, terminal=terminal)
    if with_beta and inp["beta"] is None:
        inp["beta"] = np.random.default_rng(cfg.seed + 7).uniform(
            0.2, 1.0, inp["alpha"].shape).astype(np.float32)
    mu = None if mu_null else inp["mu"]
    dt = TORCH_DT[cfg.io_dtype]
    print(f"bwd {label}{' saved' if saved else ''} B{cfg.B} T{cfg.T} H{cfg.H} d{cfg.Dk}x{cfg.Dv} {cfg.io_dtype} "
          f"mu={'no' if mu_null else 'yes'} beta={'yes' if inp['beta'] is not None else 'no'} "
          f"S0={'yes' if inp['S0'] is not None else 'no'} terminal={terminal}", flush=True)
    fargs = (to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
             to_dev(inp["alpha"]), None if mu_null else to_dev(mu), to_dev(inp["eta"]),
             to_dev(inp["S0"]), to_dev(inp["M0"]))
    Vt = None
    if saved:
        # the residuals the forward saves, then the backward that rebuilds from them
        Vt = torch.empty_like(fargs[2])
        mdn.chunk_fwd(*fargs, beta=to_dev(inp["beta"]), Vt=Vt)
    g = mdn.chunk_bwd(*fargs, to_dev(cot["dO"], dt), to_dev(cot["dS_T"]), to_dev(cot["dM_T"]),
                      beta=to_dev(inp["beta"]), Vt=Vt)
    torch.cuda.synchronize()
    mu_ref = np.zeros_like(inp["alpha"]) if mu_null else mu
    tok = lambda x: None if x is None else (x if heads is None else gather_heads(x, heads))
    st = lambda x: None if x is None else (x if heads is None else gather_heads(x, heads, True))
    ref = oracle.recurrence_backward(tok(inp["q"]), tok(inp["k"]), tok(inp["v"]),
                                     tok(inp["alpha"]), tok(mu_ref), tok(inp["eta"]),
                                     tok(inp["beta"]), st(inp["S0"]), st(inp["M0"]),
                                     dO=tok(cot["dO"]), dST=st(cot["dS_T"]),
                                     dMT=st(cot["dM_T"]))
    if heads is not None:
        for name in NAMES:
            if g[name] is not None:
                x = to_np(g[name])
                g[name] = gather_heads(x, heads, state=name in ("dS0", "dM0"))
    tol = TOL[cfg.io_dtype]
    worst = (0.0, "")
    for name in NAMES:
        x = g[name]
        r = ref[name]
        if name == "dmu" and mu_null:
            assert x is None
            continue
        if r is None:
            assert x is None, name
            continue
        x = x if isinstance(x, np.ndarray) else to_np(x)
        assert x.shape == r.shape, (name, x.shape, r.shape)
        assert np.all(np.isfinite(x)), f"{name}: non-finite values"
        err = float(np.max(np.abs(x - r))) if r.size else 0.0
        mx = float(np.max(np.abs(r))) if r.size else 0.0
        rel = err / mx if mx > 0 else err
        print(f"  {name}: max|err|={err:.3e} max|ref|={mx:.3e} rel={rel:.3e} (tol {tol})")
        worst = max(worst, (rel / tol, name))
        assert rel <= tol, f"{name}: relative error {rel:.3e} > {tol}"
    print(f"  worst ratio to the bound: {worst[0]:.3f} ({worst[1]})")


SMALL = si.CONFIGS[0]


@pytest.mark.parametrize("T", [1, 37, 64, 65, 200])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_bwd_small_fp32(T, dims):
    cfg = si.replace(SMALL, B=2, T=T, H=2, Dk=dims[0], Dv=dims[1], init_state_std=0.5,
                     seed=si.SEED_BASE + 300 + T)
    run_case(cfg, label="small")


@pytest.mark.parametrize("T", [37, 200])
def test_bwd_beta_and_no_terminal(T):
    cfg = si.replace(SMALL, B=1, T=T, H=3, Dk=64, Dv=64, seed=si.SEED_BASE + 310 + T)
    run_case(cfg, terminal=False, with_beta=True, label="beta")


@pytest.mark.parametrize("T", [37, 200])
def test_bwd_mu_null(T):
    cfg = si.replace(SMALL, B=1, T=T, H=2, Dk=64, Dv=128, init_state_std=0.3,
                     seed=si.SEED_BASE + 320 + T)
    run_case(cfg, mu_null=True, with_beta=True, label="mu0")


@pytest.mark.parametrize("T", [1, 37, 64, 65, 200])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_bwd_small_bf16(T, dims):
    cfg = si.replace(SMALL, B=1, T=T, H=2, Dk=dims[0], Dv=dims[1], io_dtype="bf16",
                     init_state_std=0.5, seed=si.SEED_BASE + 330 + T)
    run_case(cfg, label="bf16")


def test_bwd_config0():
    run_case(si.CONFIGS[0], label="config 0")


def test_bwd_no_tokens_passes_state_gradients():
    dev = "cuda"
    B, H, D = 2, 3, 64
    z = lambda *s: torch.zeros(s, device=dev)
    q = torch.zeros((B, 0, H, D), device=dev)
    dST = torch.randn((B, H, D, D), device=dev)
    dMT = torch.randn((B, H, D, D), device=dev)
    g = mdn.chunk_bwd(q, q, q, z(B, 0, H), z(B, 0, H), z(B, 0, H), None, None, q, dST, dMT)
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"], dST) and torch.equal(g["dM0"], dMT)


def test_bwd_config1_full():
    """The 400M-like layer (B4 H8 T2048 d128, bf16), every head."""
    run_case(si.CONFIGS[1], seed=11, label="config 1")


def test_bwd_config2_full():
    """The 1.3B-like layer at full size (B8 H16 T4096 d128, bf16) in one
    call, as the benchmark runs it; every head and element."""
    run_case(si.CONFIGS[2], seed=12, label="config 2 all heads")


def test_bwd_deterministic():
    cfg = si.replace(SMALL, B=2, T=200, H=3, Dk=128, Dv=128, io_dtype="bf16",
                     init_state_std=0.5, seed=si.SEED_BASE + 340)
    inp = si.make_forward(cfg)
    cot = si.backward_cotangents(cfg, 6)
    dt = TORCH_DT["bf16"]
    args = (to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
            to_dev(inp["alpha"]), to_dev(inp["mu"]), to_dev(inp["eta"]), to_dev(inp["S0"]),
            to_dev(inp["M0"]), to_dev(cot["dO"], dt), to_dev(cot["dS_T"]), to_dev(cot["dM_T"]))
    g1 = mdn.chunk_bwd(*args)
    g2 = mdn.chunk_bwd(*args)
    torch.cuda.synchronize()
    for name in NAMES:
        if g1[name] is not None:
            assert torch.equal(g1[name], g2[name]), name


@pytest.mark.parametrize("T", [37, 200])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128)])
def test_bwd_saved_residuals_fp32(T, dims):
    """The forward saves Vt (fp32 split path); the backward rebuilds the
    states from it."""
    cfg = si.replace(SMALL, B=2, T=T, H=2, Dk=dims[0], Dv=dims[1], init_state_std=0.5,
                     seed=si.SEED_BASE + 350 + T)
    run_case(cfg, label="small", saved=True)


@pytest.mark.parametrize("T", [65, 200])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("gates", ["mu", "mu0-beta"])
def test_bwd_saved_residuals_bf16(T, dims, gates):
    """The fused bf16 forward saves Vt; the backward rebuilds the states
    from it; with mu, and with no mu and a beta gate."""
    cfg = si.replace(SMALL, B=1, T=T, H=2, Dk=dims[0], Dv=dims[1], io_dtype="bf16",
                     init_state_std=0.5, seed=si.SEED_BASE + 360 + T + dims[0] + 2 * dims[1])
    if gates == "mu":
        run_case(cfg, label="bf16", saved=True)
    else:
        run_case(cfg, label="bf16 mu0 beta", saved=True, mu_null=True, with_beta=True)


def test_bwd_saved_residuals_config2_full():
    """Config 2 at full size from the forward's saved residuals, every head."""
    run_case(si.CONFIGS[2], seed=13, label="config 2 all heads", saved=True)


@pytest.mark.parametrize("io,dims,T", [("f32", (64, 64), 200), ("f32", (128, 64), 65),
                                       ("bf16", (128, 128), 200), ("bf16", (64, 128), 37)])
def test_forward_saves_residuals(io, dims, T):
    """The residuals mdn_chunk_fwd saves against the oracle's vt_t, and the
    other outputs unchanged (bitwise) by saving them.  The column tiles are
    the bf16 partition that stores residuals, so both calls run them."""
    from parity import assert_close

    cfg = si.replace(SMALL, B=2, T=T, H=3, Dk=dims[0], Dv=dims[1], io_dtype=io,
                     init_state_std=0.3, seed=si.SEED_BASE + 370 + T)
    inp = si.make_forward(cfg)
    dt = TORCH_DT[io]
    args = (to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt), to_dev(inp["alpha"]),
            to_dev(inp["mu"]), to_dev(inp["eta"]), to_dev(inp["S0"]), to_dev(inp["M0"]))
    print(f"residuals {io} d{dims} T{T}", flush=True)
    Vt = torch.empty_like(args[2])
    with mdn.fwd_path("column_tiles"):
        O1, S1, M1 = mdn.chunk_fwd(*args, Vt=Vt)
        O2, S2, M2 = mdn.chunk_fwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2) and torch.equal(M1, M2)
    _, _, _, VT = oracle.recurrence(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["mu"],
                                    inp["eta"], None, inp["S0"], inp["M0"], return_vt=True)
    if io == "f32":
        assert_close(to_np(Vt), VT, io, "Vt")
    else:
        # bf16: the residuals reach several units (v is unit scale), and storing
        # one in bf16 alone moves it by up to 2^-8 of itself; with the forward's
        # bf16-operand arithmetic: |x - x*| <= 1e-2 max|x*| (measured <= 4e-3)
        x = to_np(Vt)
        err = float(np.max(np.abs(x - VT)))
        mx = float(np.max(np.abs(VT)))
        print(f"  Vt: max|err|={err:.3e} max|ref|={mx:.3e} rel={err / mx:.3e} (tol 1e-2)")
        assert np.all(np.isfinite(x)) and err <= 1e-2 * mx
