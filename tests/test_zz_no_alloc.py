"""mdn_chunk_fwd_noalloc, the forward on the library's own per-device
scratch array (no workspace argument, no allocation), against mdn_chunk_fwd
on the same inputs: two calls in a row, the second smaller (the array keeps
the first call's contents), in bf16 under both partitions of the state (the
fused kernel's coefficient tables; the prepare kernel's T and A for the
row-split scan) and fp32 (the two-phase path's T and A), each also against
the oracle at the parity tolerances; the headline size near the array's
limit; a row split whose workspace does not fit, which runs the column tiles;
and a problem over the limit, which is refused before anything runs."""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from chunkwise_delta_rule_amd import mdn
from parity import TORCH_DT, assert_close, oracle_forward, to_dev, to_np

pytestmark = pytest.mark.gpu


def dev_args(inp, io):
    dt = TORCH_DT[io]
    return (to_dev(inp["q"], dt), to_dev(inp["k"], dt), to_dev(inp["v"], dt),
            to_dev(inp["alpha"]), to_dev(inp["mu"]), to_dev(inp["eta"]), to_dev(inp["S0"]),
            to_dev(inp["M0"]))


@pytest.mark.parametrize("io,path", [("bf16", "column_tiles"), ("bf16", "row_split"),
                                     ("f32", "auto")])
def test_noalloc_matches_chunk_fwd_twice(io, path):
    shapes = [dict(B=2, T=700, H=4), dict(B=1, T=130, H=2)]      # the second call smaller
    for n, shp in enumerate(shapes):
        cfg = dataclasses.replace(si.CONFIGS[1], io_dtype=io, Dk=64 if io == "f32" else 128,
                                  Dv=64 if io == "f32" else 128, init_state_std=0.3,
                                  seed=7100 + n, **shp)
        inp = si.make_forward(cfg)
        args = dev_args(inp, io)
        print(f"noalloc {io} {path} call {n}: B{cfg.B} T{cfg.T} H{cfg.H} d{cfg.Dk}", flush=True)
        with mdn.fwd_path(path):
            ref = mdn.chunk_fwd(*args, beta=None)
            got = mdn.chunk_fwd(*args, noalloc=True)
        torch.cuda.synchronize()
        for x, y, name in zip(got, ref, ("O", "S_T", "M_T")):
            assert torch.equal(x, y), f"{name}: noalloc differs from mdn_chunk_fwd"
        orc = oracle_forward(inp)
        for x, r, name in zip(got, orc, ("O", "S_T", "M_T")):
            assert_close(to_np(x), r, io, name)


def test_noalloc_headline_size():
    """B8 H16 T4096 d128 bf16: 54.5 MB of coefficient tables in the 64 MiB
    array; bitwise against mdn_chunk_fwd, then a small call after it."""
    inp = si.make_forward(si.CONFIGS[2])
    args = dev_args(inp, "bf16")
    del inp
    print("noalloc headline size", flush=True)
    ref = mdn.chunk_fwd(*args)
    got = mdn.chunk_fwd(*args, noalloc=True)
    torch.cuda.synchronize()
    for x, y, name in zip(got, ref, ("O", "S_T", "M_T")):
        assert torch.equal(x, y), name
    del args, ref, got
    cfg = dataclasses.replace(si.CONFIGS[1], B=1, T=77, H=3, init_state_std=0.3, seed=7200)
    inp = si.make_forward(cfg)
    args = dev_args(inp, "bf16")
    got = mdn.chunk_fwd(*args, noalloc=True)
    ref = mdn.chunk_fwd(*args)
    torch.cuda.synchronize()
    for x, y, name in zip(got, ref, ("O", "S_T", "M_T")):
        assert torch.equal(x, y), name


def test_noalloc_row_split_too_large_runs_column_tiles():
    """B1 H16 T16384 d128 under the row split: its workspace (75.5 MB) exceeds
    the 64 MiB array, so the no-alloc call runs the column tiles (27.3 MB of
    tables) and equals mdn_chunk_fwd under the column tiles bitwise."""
    cfg = si.CONFIGS[3]
    lib = mdn.load_library()
    assert lib.mdn_chunk_fwd_split_workspace_bytes(cfg.B, cfg.T, cfg.H, 128, 128, 64,
                                                   mdn.MDN_BF16) > mdn.NOALLOC_SCRATCH_BYTES
    inp = si.make_forward(cfg)
    args = dev_args(inp, "bf16")
    del inp
    print("noalloc row split over the array: B1 H16 T16384", flush=True)
    with mdn.fwd_path("row_split"):
        got = mdn.chunk_fwd(*args, noalloc=True)
    with mdn.fwd_path("column_tiles"):
        ref = mdn.chunk_fwd(*args)
    torch.cuda.synchronize()
    for x, y, name in zip(got, ref, ("O", "S_T", "M_T")):
        assert torch.equal(x, y), name


def test_noalloc_refuses_over_the_limit():
    """B8 H16 T8192 bf16 needs 109 MB of tables: MDN_ERR_WORKSPACE, nothing
    written."""
    B, T, H, D = 8, 8192, 16, 128
    lib = mdn.load_library()
    assert lib.mdn_chunk_fwd_workspace_bytes(B, T, H, D, D, 64, mdn.MDN_BF16) > \
        mdn.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    g = torch.full((B, T, H), 0.5, device="cuda")
    O = torch.full_like(x, 3.0)
    with pytest.raises(mdn.MdnError) as ex:
        mdn.chunk_fwd(x, x, x, g, g, g, O=O, noalloc=True)
    assert ex.value.status == 6
    torch.cuda.synchronize()
    assert bool((O == 3.0).all())
