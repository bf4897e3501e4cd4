"""GPU parity of the segment scan (mdn_set_fwd_path("segments")) against the
fp64 oracle, through the C ABI.

The segment scan cuts the sequence into nseg segments: segment 0 runs from
the entry state beside the state maps of the middle segments (each map
found by running the chunk recurrence from the identity's columns with
V = 0), a small kernel chains the maps into the later segments' entry
states, and a second pass runs those segments.  Every case asserts that
the shape does segment (mdn_fwd_segment_count >= 3), then compares O, S_T
and M_T element by element with the oracle at the bf16 bound of parity.py:
ragged lengths (a partial last chunk, a short last segment), every head-size
pair, nonzero entry states, mu given and mu NULL, beta, two batch rows; the
long-context layer B1 H16 T16384 d128 in full (runs A and B, and with slowly
forgetting gates); gates that forget slowly at small shapes, where the oracle
first shows that each segment's entry state moves its outputs far beyond the
bound; state passing, in-place final states, bitwise determinism, the exact
workspace, and the residual request, which the segment scan leaves to the
column tiles.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from chunkwise_delta_rule_amd import mdn
from parity import assert_close, gpu_forward, oracle_forward, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _segments():
    with mdn.fwd_path("segments"):
        yield


def check(got, ref, tag):
    print(f"[{tag}]")
    assert_close(got[0], ref[0], "bf16", "O")
    assert_close(got[1], ref[1], "bf16", "S_T")
    assert_close(got[2], ref[2], "bf16", "M_T")


def segmented(cfg, with_mu=True):
    n = mdn.segment_count(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, with_mu)
    assert n >= 3, f"{cfg} does not segment"
    return n


SMALL = [(dk, dv, T, B, H) for (dk, dv) in ((128, 128), (64, 64), (128, 64), (64, 128))
         for (T, B, H) in ((1536, 1, 2), (1601, 2, 1), (2600, 1, 3))]


@pytest.mark.parametrize("dk,dv,T,B,H", SMALL,
                         ids=[f"dk{a}-dv{b}-T{c}-B{d}-H{e}" for a, b, c, d, e in SMALL])
def test_segments_small(dk, dv, T, B, H):
    """Three to five segments; T = 1536 (24 full chunks), 1601 (a one-row
    last chunk), 2600; nonzero S0 and M0."""
    cfg = dataclasses.replace(si.CONFIGS[1], B=B, T=T, H=H, Dk=dk, Dv=dv, io_dtype="bf16",
                              init_state_std=0.3, seed=7000 + T + dk + 2 * dv + B)
    n = segmented(cfg)
    inp = si.make_forward(cfg)
    check(gpu_forward(inp), oracle_forward(inp), f"segments ({n}) dk{dk} dv{dv} T{T} B{B} H{H}")


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_segments_mu_null_and_beta(dk, dv):
    """mu NULL (the momentum-free scan: maps of S alone) against the
    oracle's mu = 0, and the four-gate form with beta."""
    cfg = dataclasses.replace(si.CONFIGS[1], B=1, T=2100, H=2, Dk=dk, Dv=dv, io_dtype="bf16",
                              init_state_std=0.3, seed=7100 + dk)
    segmented(cfg, with_mu=False)
    inp = si.make_forward(cfg)
    mu0 = np.zeros_like(inp["mu"])
    check(gpu_forward(inp, mu_null=True), oracle_forward(inp, mu=mu0), f"segments mu NULL d{dk}")
    cfgb = dataclasses.replace(cfg, beta="uniform", seed=7200 + dk)
    inpb = si.make_forward(cfgb)
    check(gpu_forward(inpb), oracle_forward(inpb), f"segments beta d{dk}")


def test_segments_long_context():
    """B1 H16 T16384 d128, every head: run A as drawn, run B with mu = 0 (mu
    given as zeros, and mu NULL), and run A's inputs with gates that forget
    slowly (alpha in [0.999, 1], eta in [0.01, 0.05])."""
    cfg = si.CONFIGS[3]
    n = segmented(cfg)
    inp = si.make_forward(cfg)
    print(f"long context, {n} segments: run A", flush=True)
    check(gpu_forward(inp), oracle_forward(inp), f"T16384 run A all heads, {n} segments")
    mu0 = np.zeros_like(inp["mu"])
    ref0 = oracle_forward(inp, mu=mu0)
    print("long context: run B", flush=True)
    check(gpu_forward(inp, mu=mu0), ref0, "T16384 run B (mu = 0) all heads")
    n0 = segmented(cfg, with_mu=False)
    check(gpu_forward(inp, mu_null=True), ref0, f"T16384 run B (mu NULL) all heads, {n0} segments")
    # The workload's gates forget a state within a segment (the result is then
    # the column tiles' bits); with gates that forget slowly every segment's
    # entry state matters, and the maps and their chain decide the result.
    rng = np.random.default_rng(cfg.seed + 1)
    slow = dict(inp)
    slow["alpha"] = rng.uniform(0.999, 1.0, size=inp["alpha"].shape).astype(np.float32)
    slow["eta"] = rng.uniform(0.01, 0.05, size=inp["eta"].shape).astype(np.float32)
    print("long context: slow gates", flush=True)
    check(gpu_forward(slow), oracle_forward(slow), f"T16384 slow gates all heads, {n} segments")


@pytest.mark.parametrize("T1", [1600, 1664])
def test_segments_state_passing(T1):
    """fwd(0:T) == fwd(T1:T | S, M from fwd(0:T1)), both halves segmented."""
    inp = si.make_forward(si.CONFIGS[1], B=1, T=3300, H=2, init_state_std=0.2, seed=7300 + T1)
    segmented(dataclasses.replace(inp["cfg"], T=T1))
    segmented(dataclasses.replace(inp["cfg"], T=3300 - T1))
    tok = ("q", "k", "v", "alpha", "mu", "eta")
    first = {key: (val[:, :T1] if key in tok else val) for key, val in inp.items()}
    second = {key: (val[:, T1:] if key in tok else val) for key, val in inp.items()}
    O1, S1, M1 = gpu_forward(first)
    O2, S2, M2 = gpu_forward(second, S0=S1.astype(np.float32), M0=M1.astype(np.float32))
    check((np.concatenate([O1, O2], axis=1), S2, M2), oracle_forward(inp),
          f"segments, state passed at T1={T1}")


def test_segments_in_place_final_state():
    """S_T may be S0 and M_T may be M0 exactly: segment 0 reads the entry
    state in the first pass, the last segment writes the exit in the second."""
    inp = si.make_forward(si.CONFIGS[1], B=1, T=1800, H=2, init_state_std=0.3, seed=7400)
    segmented(inp["cfg"])
    dt = torch.bfloat16
    S, M = to_dev(inp["S0"]), to_dev(inp["M0"])
    O, ST, MT = mdn.chunk_fwd(to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
                              to_dev(inp["alpha"]), to_dev(inp["mu"]), to_dev(inp["eta"]), S, M,
                              S_T=S, M_T=M)
    torch.cuda.synchronize()
    assert ST.data_ptr() == S.data_ptr() and MT.data_ptr() == M.data_ptr()
    check((to_np(O), to_np(S), to_np(M)), oracle_forward(inp), "segments in place")


def test_segments_deterministic():
    """Two launches on the same inputs are bitwise equal."""
    inp = si.make_forward(si.CONFIGS[1], B=1, T=2000, H=4, init_state_std=0.2, seed=7500)
    segmented(inp["cfg"])
    a = gpu_forward(inp)
    b = gpu_forward(inp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_segments_workspace():
    """The segment scan's workspace is what mdn_chunk_fwd_workspace_bytes
    reports under this setting; one byte less is refused before any launch."""
    B, T, H, D = 1, 2000, 4, 128
    need = mdn.workspace_bytes(B, T, H, D, D, torch.bfloat16)
    with mdn.fwd_path("column_tiles"):
        fused = mdn.workspace_bytes(B, T, H, D, D, torch.bfloat16)
    assert need > fused
    inp = si.make_forward(si.CONFIGS[1], B=B, T=T, H=H, seed=7600)
    dt = torch.bfloat16
    args = [to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
            to_dev(inp["alpha"]), to_dev(inp["mu"]), to_dev(inp["eta"]), None, None]
    ws = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(mdn.MdnError, match="WORKSPACE"):
        mdn.chunk_fwd(*args, workspace=ws)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    O, ST, MT = mdn.chunk_fwd(*args, workspace=ws)
    torch.cuda.synchronize()
    check((to_np(O), to_np(ST), to_np(MT)), oracle_forward(inp), "segments, exact workspace")


def test_segments_with_residuals_run_the_column_tiles():
    """A call that asks for the residuals Vt runs the column tiles (the
    segment scan stores none) and still matches the oracle."""
    inp = si.make_forward(si.CONFIGS[1], B=1, T=1700, H=2, init_state_std=0.2, seed=7700)
    segmented(inp["cfg"])
    dt = torch.bfloat16
    Vt = torch.empty((1, 1700, 2, 128), dtype=dt, device="cuda")
    O, ST, MT = mdn.chunk_fwd(to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
                              to_dev(inp["alpha"]), to_dev(inp["mu"]), to_dev(inp["eta"]),
                              to_dev(inp["S0"]), to_dev(inp["M0"]), Vt=Vt)
    torch.cuda.synchronize()
    assert float(Vt.float().abs().max()) > 0
    check((to_np(O), to_np(ST), to_np(MT)), oracle_forward(inp), "segments + Vt")


def test_segments_plan():
    """mdn.ChunkPlan (fixed buffers, as the benchmark times them) under the
    segment scan, where its workspace exceeds the two phases' (B4 H8 T2048:
    3 segments), gives the same bits as a plain call."""
    inp = si.make_forward(si.CONFIGS[1], seed=7800)
    cfg = inp["cfg"]
    segmented(cfg)
    assert mdn.workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, torch.bfloat16) > \
        mdn.workspace_bytes(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, torch.bfloat16, split=True)
    dt = torch.bfloat16
    args = (to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt), to_dev(inp["alpha"]),
            to_dev(inp["mu"]), to_dev(inp["eta"]), to_dev(inp["S0"]), to_dev(inp["M0"]))
    plan = mdn.ChunkPlan(*args)
    plan.forward()
    O, ST, MT = mdn.chunk_fwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(plan.O, O) and torch.equal(plan.S_T, ST) and torch.equal(plan.M_T, MT)


CARRY = [(dk, dv, mu_null) for (dk, dv) in ((128, 128), (64, 64), (128, 64)) for mu_null in (False, True)]


@pytest.mark.parametrize("dk,dv,mu_null", CARRY,
                         ids=[f"dk{a}-dv{b}-{'mu_null' if c else 'mu'}" for a, b, c in CARRY])
def test_segments_carry_across_segments(dk, dv, mu_null):
    """Gates that forget slowly (alpha in [0.999, 1], eta in [0.01, 0.05]),
    so that every segment's entry state shapes its outputs: the state maps
    and their chain decide the result.  With the workload's own gates a
    state fades within a segment and the segment scan gives the column
    tiles' bits.  The oracle first shows that dropping the entry state of
    the segments after the first changes their outputs by far more than the
    bound; then the GPU matches the oracle, and differs from the column
    tiles only by rounding."""
    cfg = dataclasses.replace(si.CONFIGS[1], B=1, T=2600, H=2, Dk=dk, Dv=dv, io_dtype="bf16",
                              init_state_std=0.3, seed=7900 + dk + dv + int(mu_null))
    n = segmented(cfg, with_mu=not mu_null)
    inp = si.make_forward(cfg)
    rng = np.random.default_rng(cfg.seed)
    inp["alpha"] = rng.uniform(0.999, 1.0, size=inp["alpha"].shape).astype(np.float32)
    inp["eta"] = rng.uniform(0.01, 0.05, size=inp["eta"].shape).astype(np.float32)
    mu = np.zeros_like(inp["mu"]) if mu_null else None
    ref = oracle_forward(inp, mu=mu)
    # the tail from the second segment on, run from a zero state instead
    nc = -(-cfg.T // 64)
    t1 = 64 * -(-nc // n)
    tok = ("q", "k", "v", "alpha", "mu", "eta")
    tail = {key: (val[:, t1:] if key in tok else None if key in ("S0", "M0") else val)
            for key, val in inp.items()}
    tail_ref = oracle_forward(tail, mu=None if mu is None else mu[:, t1:])
    gap = float(np.abs(tail_ref[0] - ref[0][:, t1:]).max())
    print(f"[carry, {n} segments] dropping the entry at token {t1} moves O by {gap:.3e}")
    assert gap > 0.1
    got = gpu_forward(inp, mu_null=mu_null)
    check(got, ref, f"segments ({n}), slow gates, dk{dk} dv{dv}{' mu NULL' if mu_null else ''}")
    with mdn.fwd_path("column_tiles"):
        tiles = gpu_forward(inp, mu_null=mu_null)
    for name, a, b in zip(("O", "S_T", "M_T"), got, tiles):
        d = float(np.abs(a.astype(np.float64) - b).max())
        print(f"  {name} segments vs column tiles: {d:.3e}")
        assert d <= 2e-2 * max(1.0, float(np.abs(b).max()))
