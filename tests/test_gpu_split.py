"""GPU parity of the split entry points (mdn_chunk_fwd_prepare followed by
mdn_chunk_fwd_scan, through the C ABI) against the fp64 oracle.  For bf16
inputs these run a different pair of kernels from mdn_chunk_fwd's fused one,
so they get their own cases; tolerances are in parity.py."""
import dataclasses

import pytest

import synthetic_inputs as si
from parity import assert_close, gpu_forward, oracle_forward, split_forward

pytestmark = pytest.mark.gpu


def check(io, got, ref, tag):
    print(f"[{tag}]")
    for x, r, name in zip(got, ref, ("O", "S_T", "M_T")):
        assert_close(x, r, io, name)


CASES = [(io, dk, dv, T) for io in ("bf16", "f32") for (dk, dv) in ((64, 128), (128, 128))
         for T in (1, 65, 200)]


@pytest.mark.parametrize("io,dk,dv,T", CASES, ids=[f"{a}-dk{b}-dv{c}-T{d}" for a, b, c, d in CASES])
def test_split_small_shapes(io, dk, dv, T):
    cfg = dataclasses.replace(si.CONFIGS[1], B=2, T=T, H=3, Dk=dk, Dv=dv, io_dtype=io,
                              init_state_std=0.3, seed=2000 + T + dk + 2 * dv)
    inp = si.make_forward(cfg)
    check(io, split_forward(inp), oracle_forward(inp), f"split {io} dk{dk} dv{dv} T{T}")


def test_split_400m_like_layer():
    inp = si.make_forward(si.CONFIGS[1])
    check("bf16", split_forward(inp), oracle_forward(inp), "split B4H8T2048d128")


def test_split_and_fused_agree():
    """Both bf16 paths evaluate the same chunk equations: their difference is
    rounding, bounded by the parity tolerance of each against the oracle."""
    inp = si.make_forward(si.CONFIGS[1], B=2, T=700, H=4, init_state_std=0.3, seed=91)
    a, b = split_forward(inp), gpu_forward(inp)
    for x, y, name in zip(a, b, ("O", "S_T", "M_T")):
        assert_close(x, y, "bf16", f"split vs fused {name}")
