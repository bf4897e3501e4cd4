"""GPU parity of mdn_chunk_fwd against the fp64 oracle, through the C ABI.

Sizes: every config in full (the fp32 case, the 400M-like layer, the
headline 1.3B-like layer in the launch configuration the benchmark times,
both long-context runs), every element against the oracle, plus many small
ragged shapes.  Every bf16 case runs under both partitions of the state
(mdn_set_fwd_path): the column tiles (one fused kernel) and the row split
(the prepare kernel, then the row-split scan); the default rule picks one of
them by size, so both are the product path.  Tolerances are in parity.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from chunkwise_delta_rule_amd import mdn
from parity import (TORCH_DT, assert_close, gather_heads, gpu_forward, oracle_forward,
                    split_forward, to_dev, to_np)

pytestmark = pytest.mark.gpu

PATHS = ("column_tiles", "row_split")


@pytest.fixture(autouse=True)
def _forward_path(request):
    """A test parametrized over `path` runs under that partition of the bf16
    forward's state; the others under the default rule."""
    spec = getattr(request.node, "callspec", None)
    path = spec.params.get("path", "auto") if spec is not None else "auto"
    with mdn.fwd_path(path):
        yield


_REF = {}


def cached_oracle(config, variant, inp, **kw):
    """Oracle results of one full-size config, kept while the tests of that
    config run under each path."""
    if any(key[0] != config for key in _REF):
        _REF.clear()
    if (config, variant) not in _REF:
        _REF[(config, variant)] = oracle_forward(inp, **kw)
    return _REF[(config, variant)]


def io_paths(ios):
    """(io, path) pairs: bf16 under both partitions, fp32 (one path) once."""
    return [(io, p) for io in ios for p in (PATHS if io == "bf16" else ("auto",))]


def check_all(io, got, ref, tag, pairs=None):
    O, ST, MT = got
    if pairs is not None:
        O = gather_heads(O, pairs)
        ST = gather_heads(ST, pairs, True)
        MT = gather_heads(MT, pairs, True)
    print(f"[{tag}]")
    assert_close(O, ref[0], io, "O")
    assert_close(ST, ref[1], io, "S_T")
    assert_close(MT, ref[2], io, "M_T")


def test_fp32_config():
    """B1 H2 T256 d64, fp32 I/O: 1e-4 relative on O, S_T and M_T."""
    inp = si.make_forward(si.CONFIGS[0])
    check_all("f32", gpu_forward(inp), oracle_forward(inp), "fp32 B1H2T256d64")


SMALL = [(io, dk, dv, T, p) for io, p in io_paths(("f32", "bf16")) for (dk, dv) in
         ((64, 64), (64, 128), (128, 64), (128, 128)) for T in (1, 37, 64, 65, 200)]


@pytest.mark.parametrize("io,dk,dv,T,path", SMALL,
                         ids=[f"{a}-dk{b}-dv{c}-T{d}-{e}" for a, b, c, d, e in SMALL])
def test_small_shapes_with_initial_state(io, dk, dv, T, path):
    """Ragged T (a single token, partial and exact chunks, several tiles),
    every supported head-size pair, nonzero S0 and M0."""
    cfg = dataclasses.replace(si.CONFIGS[1], B=2, T=T, H=3, Dk=dk, Dv=dv, io_dtype=io,
                              init_state_std=0.3, seed=1000 + T + dk + 2 * dv)
    inp = si.make_forward(cfg)
    check_all(io, gpu_forward(inp), oracle_forward(inp), f"{io} dk{dk} dv{dv} T{T}")


@pytest.mark.parametrize("path", PATHS)
def test_more_heads_than_one_coefficient_group(path):
    """H = 20 with bf16 I/O: the coefficient tables are built 16 heads per
    workgroup, so this takes a full and a partial head group; ragged T."""
    cfg = dataclasses.replace(si.CONFIGS[1], B=2, T=130, H=20, Dk=64, Dv=64, io_dtype="bf16",
                              init_state_std=0.3, seed=4242)
    inp = si.make_forward(cfg)
    check_all("bf16", gpu_forward(inp), oracle_forward(inp), "bf16 B2 H20 T130 d64")


BETA = [(io, dk, dv, T, p) for io, p in io_paths(("f32", "bf16"))
        for (dk, dv) in ((64, 64), (128, 128)) for T in (37, 200)]


@pytest.mark.parametrize("io,dk,dv,T,path", BETA,
                         ids=[f"{a}-dk{b}-dv{c}-T{d}-{e}" for a, b, c, d, e in BETA])
def test_beta_gate(io, dk, dv, T, path):
    """The four-gate form: an explicit update-step gate beta (uniform in
    [0.2, 1]) against the oracle's beta recurrence; ragged T, nonzero S0, M0."""
    cfg = dataclasses.replace(si.CONFIGS[1], B=2, T=T, H=3, Dk=dk, Dv=dv, io_dtype=io,
                              init_state_std=0.3, beta="uniform", seed=5000 + T + dk + dv)
    inp = si.make_forward(cfg)
    check_all(io, gpu_forward(inp), oracle_forward(inp), f"beta {io} dk{dk} dv{dv} T{T}")


@pytest.mark.parametrize("path", PATHS)
def test_beta_gate_split_phases(path):
    """beta through the two exported phases (prepare, then scan) in bf16."""
    cfg = dataclasses.replace(si.CONFIGS[1], B=1, T=150, H=4, io_dtype="bf16",
                              init_state_std=0.3, beta="logit", seed=5555)
    inp = si.make_forward(cfg)
    check_all("bf16", split_forward(inp), oracle_forward(inp), "beta split bf16")


@pytest.mark.parametrize("io,path", io_paths(("f32", "bf16")))
def test_beta_ones_matches_no_beta_bitwise(io, path):
    """An all-ones beta runs exactly the arithmetic of no beta (both bf16
    paths and the fp32 one)."""
    cfg = dataclasses.replace(si.CONFIGS[1], B=1, T=130, H=2, io_dtype=io, init_state_std=0.3,
                              seed=5600)
    inp = si.make_forward(cfg)
    a = gpu_forward(inp, beta=None)
    b = gpu_forward(inp, beta=np.ones_like(inp["alpha"]))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("io,path", io_paths(("f32", "bf16")))
def test_mu_null_runs_the_gated_delta_rule(io, path):
    """No mu (mu = 0): the momentum-free kernels (bf16) and the split path
    (fp32) against the oracle at mu = 0, with S0 and M0 given (M0 is not
    read: a NaN M0 must not show) and a beta gate; M_T is the last token's
    own write."""
    cfg = dataclasses.replace(si.CONFIGS[1], B=2, T=150, H=3, io_dtype=io, init_state_std=0.3,
                              beta="uniform", seed=5700)
    inp = si.make_forward(cfg)
    mu0 = np.zeros_like(inp["mu"])
    got = gpu_forward(inp, mu_null=True, M0=np.full_like(inp["M0"], np.nan))
    check_all(io, got, oracle_forward(inp, mu=mu0), f"mu NULL {io}")
    # against the general kernel given mu = 0 explicitly
    ref = gpu_forward(inp, mu=mu0)
    for x, y, name in zip(got, ref, ("O", "S_T", "M_T")):
        assert_close(x, y, io, name + " (mu NULL vs mu = 0)")


@pytest.mark.parametrize("path", PATHS)
def test_mu_null_split_phases(path):
    """No mu through the exported phases in bf16."""
    cfg = dataclasses.replace(si.CONFIGS[1], B=1, T=100, H=4, io_dtype="bf16",
                              init_state_std=0.3, seed=5800)
    inp = si.make_forward(cfg)
    check_all("bf16", split_forward(inp, mu_null=True),
              oracle_forward(inp, mu=np.zeros_like(inp["mu"])), "mu NULL split bf16")


@pytest.mark.parametrize("path", PATHS)
def test_gated_delta_rule_special_case(path):
    """mu = 0 exactly: the operator is the gated delta rule; the final
    momentum is then rank one, -eta_T k_T vt_T^T (checked on the oracle side
    by its pins), and the GPU matches the oracle at mu = 0."""
    inp = si.make_forward(si.CONFIGS[1], B=1, T=333, H=4, init_state_std=0.3, seed=77)
    mu0 = np.zeros_like(inp["mu"])
    got = gpu_forward(inp, mu=mu0)
    ref = oracle_forward(inp, mu=mu0)
    check_all("bf16", got, ref, "mu=0")
    # rank one final momentum on the GPU too
    for h in range(4):
        sv = np.linalg.svd(got[2][0, h], compute_uv=False)
        assert sv[1] <= 1e-2 * sv[0]


@pytest.mark.parametrize("path", PATHS)
def test_delta_rule_special_case(path):
    """alpha = 1, mu = 0: DeltaNet with write strength eta."""
    inp = si.make_forward(si.CONFIGS[1], B=1, T=200, H=2, seed=78)
    inp["alpha"] = np.ones_like(inp["alpha"])
    mu0 = np.zeros_like(inp["mu"])
    check_all("bf16", gpu_forward(inp, mu=mu0), oracle_forward(inp, mu=mu0), "alpha=1 mu=0")


@pytest.mark.parametrize("path", PATHS)
def test_400m_like_layer_full(path):
    """B4 H8 T2048 d128, bf16 I/O, every head against the oracle."""
    inp = si.make_forward(si.CONFIGS[1])
    check_all("bf16", gpu_forward(inp), cached_oracle("400m", "A", inp),
              f"bf16 B4H8T2048d128 {path}")


@pytest.mark.parametrize("path", PATHS)
def test_headline_layer_full(path):
    """B8 H16 T4096 d128 (the benchmarked launch runs the column tiles),
    every head and element against the oracle."""
    inp = si.make_forward(si.CONFIGS[2])
    print(f"headline layer B8 H16 T4096 d128 {path}: GPU", flush=True)
    got = gpu_forward(inp)
    print("headline layer: oracle", flush=True)
    check_all("bf16", got, cached_oracle("1.3b", "A", inp), f"bf16 B8H16T4096d128 all heads {path}")


@pytest.mark.parametrize("path", PATHS)
def test_long_context_and_mu_zero_run(path):
    """B1 H16 T16384 d128, every head: run A as drawn; run B with mu = 0 on
    the same inputs, both through the general kernel (mu given as zeros) and
    the momentum-free one (mu NULL); plus an independent single-state
    gated-delta-rule loop for one head of run B.  (The benchmarked launch
    runs the row split.)"""
    inp = si.make_forward(si.CONFIGS[3])
    print(f"long context B1 H16 T16384 d128 {path}: run A", flush=True)
    got = gpu_forward(inp)
    check_all("bf16", got, cached_oracle("16k", "A", inp), f"T16384 run A all heads {path}")
    mu0 = np.zeros_like(inp["mu"])
    print("long context: run B", flush=True)
    ref0 = cached_oracle("16k", "B", inp, mu=mu0)
    got0 = gpu_forward(inp, mu=mu0)
    check_all("bf16", got0, ref0, "T16384 run B (mu = 0) all heads")
    gotn = gpu_forward(inp, mu_null=True)
    check_all("bf16", gotn, ref0, "T16384 run B (mu NULL) all heads")
    # independent gated delta rule on head 3: S = aS + e k (v - a S^T k)^T
    h = 3
    q, k, v = (inp[x][0, :, h].astype(np.float64) for x in ("q", "k", "v"))
    a, e = inp["alpha"][0, :, h].astype(np.float64), inp["eta"][0, :, h].astype(np.float64)
    S = np.zeros((128, 128))
    O = np.zeros((q.shape[0], 128))
    for t in range(q.shape[0]):
        S = a[t] * S + e[t] * np.outer(k[t], v[t] - a[t] * (S.T @ k[t]))
        O[t] = S.T @ q[t]
    print("[T16384 run B vs independent gated delta rule, head 3]")
    assert_close(got0[0][0, :, h], O, "bf16", "O")
    assert_close(got0[1][0, h], S, "bf16", "S_T")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T1", [64, 100, 1000])
def test_state_passing(T1, path):
    """fwd(0:T) == fwd(T1:T | S, M from fwd(0:T1)), split on and off chunk
    boundaries; both halves also match the oracle."""
    inp = si.make_forward(si.CONFIGS[1], B=2, T=1500, H=2, init_state_std=0.2, seed=300 + T1)
    full = gpu_forward(inp)
    first = {key: (val[:, :T1] if key in ("q", "k", "v", "alpha", "mu", "eta") else val)
             for key, val in inp.items()}
    second = {key: (val[:, T1:] if key in ("q", "k", "v", "alpha", "mu", "eta") else val)
              for key, val in inp.items()}
    O1, S1, M1 = gpu_forward(first)
    O2, S2, M2 = gpu_forward(second, S0=S1.astype(np.float32), M0=M1.astype(np.float32))
    ref = oracle_forward(inp)
    print(f"[state passing at T1={T1}]")
    assert_close(np.concatenate([O1, O2], axis=1), ref[0], "bf16", "O (split)")
    assert_close(S2, ref[1], "bf16", "S_T (split)")
    assert_close(M2, ref[2], "bf16", "M_T (split)")
    assert_close(np.concatenate([O1, O2], axis=1), full[0], "bf16", "O split vs whole")


@pytest.mark.parametrize("path", PATHS)
def test_deterministic(path):
    """Two launches on the same inputs are bitwise equal."""
    inp = si.make_forward(si.CONFIGS[1], B=2, T=700, H=4, init_state_std=0.2, seed=5)
    a = gpu_forward(inp)
    b = gpu_forward(inp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("path", PATHS)
def test_in_place_final_state(path):
    """S_T may be S0 and M_T may be M0 exactly."""
    inp = si.make_forward(si.CONFIGS[1], B=1, T=190, H=2, init_state_std=0.3, seed=6)
    dt = torch.bfloat16
    S = to_dev(inp["S0"])
    M = to_dev(inp["M0"])
    O, ST, MT = mdn.chunk_fwd(to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
                              to_dev(inp["alpha"]), to_dev(inp["mu"]), to_dev(inp["eta"]), S, M,
                              S_T=S, M_T=M)
    torch.cuda.synchronize()
    assert ST.data_ptr() == S.data_ptr() and MT.data_ptr() == M.data_ptr()
    check_all("bf16", (to_np(O), to_np(S), to_np(M)), oracle_forward(inp), "in place")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("with_state", [False, True])
def test_empty_sequence(with_state, path):
    """T = 0: no tokens; the final state is the initial state (zero if absent)."""
    B, H, D = 2, 3, 128
    dt = torch.bfloat16
    q = torch.empty((B, 0, H, D), dtype=dt, device="cuda")
    g = torch.empty((B, 0, H), dtype=torch.float32, device="cuda")
    S0 = torch.randn(B, H, D, D, device="cuda") if with_state else None
    M0 = torch.randn(B, H, D, D, device="cuda") if with_state else None
    O, ST, MT = mdn.chunk_fwd(q, q, q, g, g, g, S0, M0)
    torch.cuda.synchronize()
    assert O.shape == (B, 0, H, D)
    if with_state:
        assert torch.equal(ST, S0) and torch.equal(MT, M0)
    else:
        assert torch.count_nonzero(ST) == 0 and torch.count_nonzero(MT) == 0


def test_bad_arguments_raise():
    inp = si.make_forward(si.CONFIGS[1], B=1, T=64, H=1)
    dt = torch.bfloat16
    q = to_dev(inp["q"], dt)
    g = to_dev(inp["alpha"])
    with pytest.raises(mdn.MdnError) as ex:
        mdn.chunk_fwd(q, q, q, g, g, g, O=q)           # output over the inputs
    assert ex.value.status == 5
    # a workspace smaller than mdn_chunk_fwd_workspace_bytes is refused
    qf = to_dev(inp["q"], torch.float32)
    with pytest.raises(mdn.MdnError) as ex:
        mdn.chunk_fwd(qf, qf, qf, g, g, g, workspace=torch.empty(16, dtype=torch.uint8,
                                                                device="cuda"))
    assert ex.value.status == 6
