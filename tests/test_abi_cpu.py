"""Host-side checks of the libmdn C ABI that need no GPU: the library loads,
exports every function include/libmdn.h declares, and rejects bad arguments
with the documented status before anything is launched.  Pointers here are
fake integers: every call below fails (or returns early) in host-side
validation, so no HIP call is ever made.
"""
import ctypes
import os
import re

import pytest

from chunkwise_delta_rule_amd import mdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmdn.h")


@pytest.fixture(scope="module")
def lib():
    return mdn.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mdn_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(mdn.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for code, name in mdn.STATUS_NAMES.items():
        assert lib.mdn_status_string(code).decode().startswith(name)
    assert lib.mdn_status_string(99) == b"unknown mdn_status"


def test_workspace_bytes(lib):
    ws = lib.mdn_chunk_fwd_workspace_bytes
    split = lib.mdn_chunk_fwd_split_workspace_bytes
    # per chunk: T and A (C x C in the I/O dtype) and 8 coefficient vectors
    per_bf16 = 2 * 64 * 64 * 2 + 8 * 64 * 4
    per_f32 = 2 * 64 * 64 * 4 + 8 * 64 * 4
    assert split(8, 4096, 16, 128, 128, 64, mdn.MDN_BF16) == 8 * 16 * 64 * per_bf16
    assert split(1, 65, 2, 64, 64, 64, mdn.MDN_F32) == 2 * 2 * per_f32     # ragged: 2 chunks
    assert split(1, 1, 1, 64, 128, 64, mdn.MDN_BF16) == per_bf16
    # the bf16 column tiles keep T and A on chip and need only per-chunk
    # coefficient tables (gates, block products, boundary values, Gamma's
    # diagonal blocks packed to their lower triangles, six coefficient rows:
    # 1664 floats); fp32 and the bf16 row split use the split workspace.  Under
    # MDN_FWD_AUTO the row split runs up to 32 tiles of 64 value columns.
    assert mdn.ROW_SPLIT_MAX_TILES == 32
    per_fused = 1664 * 4
    assert ws(8, 4096, 16, 128, 128, 64, mdn.MDN_BF16) == 8 * 16 * 64 * per_fused   # 256 tiles
    assert ws(1, 64, 33, 128, 64, 64, mdn.MDN_BF16) == 33 * per_fused                # 33 tiles
    assert ws(2, 64, 8, 128, 128, 64, mdn.MDN_BF16) == 16 * per_bf16                 # 32 tiles
    assert ws(1, 65, 2, 64, 64, 64, mdn.MDN_BF16) == 2 * 2 * per_bf16
    assert ws(1, 65, 2, 64, 64, 64, mdn.MDN_F32) == 2 * 2 * per_f32
    prev = lib.mdn_set_fwd_path(mdn.FWD_PATHS["column_tiles"])
    try:
        assert prev == mdn.FWD_PATHS["auto"]
        assert ws(1, 65, 2, 64, 64, 64, mdn.MDN_BF16) == 2 * 2 * per_fused
        assert ws(1, 65, 2, 64, 64, 64, mdn.MDN_F32) == 2 * 2 * per_f32
        assert lib.mdn_set_fwd_path(mdn.FWD_PATHS["row_split"]) == mdn.FWD_PATHS["column_tiles"]
        assert ws(8, 4096, 16, 128, 128, 64, mdn.MDN_BF16) == 8 * 16 * 64 * per_bf16
        assert lib.mdn_set_fwd_path(5) == -1          # unknown: nothing changes
        assert ws(8, 4096, 16, 128, 128, 64, mdn.MDN_BF16) == 8 * 16 * 64 * per_bf16
    finally:
        lib.mdn_set_fwd_path(prev)
    for bad in [(0, 64, 1, 64, 64, 64, 1), (1, 0, 1, 64, 64, 64, 1), (1, 64, 1, 96, 64, 64, 1),
                (1, 64, 1, 64, 64, 32, 1), (1, 64, 1, 64, 64, 64, 7), (-1, 64, 1, 64, 64, 64, 1)]:
        assert ws(*bad) == 0
        assert split(*bad) == 0


def test_segment_scan_choice_and_workspace(lib):
    """The segment scan's size rule (mdn_fwd_segment_count) and workspace.
    nseg is the largest count of segments, 3 or more, with both passes in one
    round of 256 workgroups -- pass 1: the heads' Dv/64 tiles plus nseg - 2
    transitions of Dv/64 + 2 Dk/64 tiles (Dk/64 without mu), pass 2: nseg - 1
    segments' tiles -- and ceil(NC / nseg) >= 16 chunks per segment under
    MDN_FWD_AUTO (>= 8 with mu NULL), >= 8 under MDN_FWD_SEGMENTS.  Its workspace: the
    coefficient tables (1664 floats per chunk), entry states of every segment
    (S and M), exit states of the nseg - 2 transitions (S and M, Dv + 2 Dk
    columns, Dv + Dk without mu), fp32."""
    count = lib.mdn_fwd_segment_count
    ws = lib.mdn_chunk_fwd_workspace_bytes
    assert count(1, 16384, 16, 128, 128, 1) == 4      # 32 + 2 * 96 = 224 workgroups
    assert count(1, 16384, 16, 128, 128, 0) == 5      # 32 + 3 * 64 = 224
    assert count(4, 2048, 8, 128, 128, 1) == 0        # 3 segments of 11 chunks: auto declines
    assert count(4, 2048, 8, 128, 128, 0) == 3        # ... but not without mu
    assert count(1, 2048, 16, 128, 128, 1) == 0
    assert count(1, 2048, 16, 128, 128, 0) == 4        # 4 segments of 8 chunks without mu
    assert count(1, 1024, 16, 128, 128, 0) == 0        # 16 chunks: too few for 3 segments of 8
    assert count(8, 4096, 16, 128, 128, 1) == 0       # 256 tiles
    assert count(1, 65536, 2, 128, 128, 1) == 23      # 4 + 21 * 12 = 256
    assert count(1, 16384, 16, 128, 128, 1) == lib.mdn_fwd_segment_count(1, 16384, 16, 128, 128, 1)
    nc, ctab = 256, 16 * 256 * 1664 * 4
    seg_mu = ctab + 2 * 4 * 16 * 128 * 128 * 4 + 2 * 2 * 16 * 128 * 384 * 4
    seg_nomu = ctab + 2 * 5 * 16 * 128 * 128 * 4 + 2 * 3 * 16 * 128 * 256 * 4
    assert ws(1, 64 * nc, 16, 128, 128, 64, mdn.MDN_BF16) == max(seg_mu, seg_nomu)
    prev = lib.mdn_set_fwd_path(mdn.FWD_PATHS["segments"])
    try:
        assert count(4, 2048, 8, 128, 128, 1) == 3    # 3 segments of 11 chunks
        assert count(1, 1536, 2, 128, 128, 1) == 3    # 3 of 8
        assert count(1, 1345, 2, 128, 128, 1) == 3    # 22 chunks (the last one row): 8, 8, 6
        assert count(1, 1344, 2, 128, 128, 1) == 0    # 21 chunks: 7 per segment
        assert count(1, 16384, 16, 128, 128, 1) == 4
        assert count(1, 16384, 16, 64, 64, 1) == 7    # 16 + 5 * 48 = 256
        assert ws(1, 64 * nc, 16, 128, 128, 64, mdn.MDN_BF16) == max(seg_mu, seg_nomu)
        # where it does not apply, the column tiles' workspace
        assert ws(8, 4096, 16, 128, 128, 64, mdn.MDN_BF16) == 8 * 16 * 64 * 1664 * 4
    finally:
        lib.mdn_set_fwd_path(prev)
    for path in ("column_tiles", "row_split"):
        prev = lib.mdn_set_fwd_path(mdn.FWD_PATHS[path])
        try:
            assert count(1, 16384, 16, 128, 128, 1) == 0
        finally:
            lib.mdn_set_fwd_path(prev)
    for bad in [(0, 4096, 1, 128, 128, 1), (1, -5, 1, 128, 128, 1), (1, 4096, 1, 96, 128, 1)]:
        assert count(*bad) == 0


# fake, 16-byte aligned, non-overlapping "device" addresses
BASE = 1 << 40
STEP = 1 << 32


def fake(i, off=0):
    return BASE + i * STEP + off


def fwd_args(**over):
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), mu=fake(4), eta=fake(5), beta=None,
             S0=fake(6), M0=fake(7), O=fake(8), Vt=None, S_T=fake(9), M_T=fake(10), B=2, T=100,
             H=3, Dk=64, Dv=128, chunk=64, dt=mdn.MDN_BF16, ws=fake(11), wsb=1 << 31,
             stream=None)
    a.update(over)
    return a


def call_fwd(lib, a):
    return lib.mdn_chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["mu"], a["eta"], a["beta"],
                             a["S0"], a["M0"], a["O"], a["Vt"], a["S_T"], a["M_T"], a["B"], a["T"],
                             a["H"], a["Dk"], a["Dv"], a["chunk"], a["dt"], a["ws"], a["wsb"],
                             a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(Dk=96), "MDN_ERR_UNSUPPORTED"),
    (dict(Dv=256), "MDN_ERR_UNSUPPORTED"),
    (dict(chunk=32), "MDN_ERR_UNSUPPORTED"),
    (dict(dt=5), "MDN_ERR_UNSUPPORTED"),
    (dict(B=-1), "MDN_ERR_SHAPE"),
    (dict(T=-5), "MDN_ERR_SHAPE"),
    (dict(q=None), "MDN_ERR_NULL"),
    (dict(eta=None), "MDN_ERR_NULL"),
    (dict(O=None), "MDN_ERR_NULL"),
    (dict(k=fake(1, 8)), "MDN_ERR_ALIGN"),
    (dict(S_T=fake(9, 4)), "MDN_ERR_ALIGN"),
    (dict(ws=None, dt=mdn.MDN_F32), "MDN_ERR_WORKSPACE"),
    (dict(wsb=1000, dt=mdn.MDN_F32), "MDN_ERR_WORKSPACE"),
    (dict(ws=None), "MDN_ERR_WORKSPACE"),
    (dict(wsb=1000), "MDN_ERR_WORKSPACE"),
    (dict(O=fake(0)), "MDN_ERR_ALIAS"),                 # output over q
    (dict(O=fake(2, 4096)), "MDN_ERR_ALIAS"),           # output inside v
    (dict(ws=fake(8), dt=mdn.MDN_F32), "MDN_ERR_ALIAS"),  # workspace over output
    (dict(S_T=fake(7)), "MDN_ERR_ALIAS"),               # final memory over initial momentum
    (dict(S_T=fake(6, 16)), "MDN_ERR_ALIAS"),           # shifted, not exactly in place
    (dict(M_T=fake(9)), "MDN_ERR_ALIAS"),               # both final states at one address
    (dict(beta=fake(12, 8)), "MDN_ERR_ALIGN"),          # the optional gate is checked too
    (dict(mu=None, M0=None, k=fake(1, 8)), "MDN_ERR_ALIGN"),  # NULL mu (mu = 0) is allowed
    (dict(beta=fake(8)), "MDN_ERR_ALIAS"),              # output over beta
    (dict(beta=fake(12), M_T=fake(12)), "MDN_ERR_ALIAS"),  # final momentum over beta
    (dict(Vt=fake(13, 8)), "MDN_ERR_ALIGN"),            # the optional residual output
    (dict(Vt=fake(8)), "MDN_ERR_ALIAS"),                # residuals over O
    (dict(Vt=fake(2)), "MDN_ERR_ALIAS"),                # residuals over v
])
def test_chunk_fwd_rejects(lib, over, status):
    assert mdn.STATUS_NAMES[call_fwd(lib, fwd_args(**over))] == status


def test_chunk_fwd_beta_is_optional(lib):
    # a NULL beta (the default above) and a valid one both pass validation;
    # B = 0 keeps the calls from launching anything
    assert call_fwd(lib, fwd_args(B=0)) == 0
    assert call_fwd(lib, fwd_args(B=0, beta=fake(12))) == 0


def test_chunk_fwd_no_work_returns_ok_without_launch(lib):
    # B = 0 or H = 0: nothing to do; pointers are never touched
    assert call_fwd(lib, fwd_args(B=0, q=None, O=None, ws=None)) == 0
    assert call_fwd(lib, fwd_args(H=0, q=None, O=None, ws=None)) == 0


def dec_args(**over):
    a = dict(q=fake(0), k=fake(1), v=fake(2), alpha=fake(3), mu=fake(4), eta=fake(5), beta=None,
             S=fake(6), M=fake(7), o=fake(8), N=4, H=2, Dk=128, Dv=128, dt=mdn.MDN_BF16,
             stream=None)
    a.update(over)
    return a


def call_dec(lib, a):
    return lib.mdn_decode_step(a["q"], a["k"], a["v"], a["alpha"], a["mu"], a["eta"], a["beta"],
                               a["S"], a["M"], a["o"], a["N"], a["H"], a["Dk"], a["Dv"], a["dt"],
                               a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(Dk=32), "MDN_ERR_UNSUPPORTED"),
    (dict(dt=2), "MDN_ERR_UNSUPPORTED"),
    (dict(N=-1), "MDN_ERR_SHAPE"),
    (dict(S=None), "MDN_ERR_NULL"),
    (dict(o=None), "MDN_ERR_NULL"),
    (dict(v=fake(2, 2)), "MDN_ERR_ALIGN"),
    (dict(o=fake(0)), "MDN_ERR_ALIAS"),
    (dict(M=fake(6, 1024)), "MDN_ERR_ALIAS"),
    (dict(S=fake(1)), "MDN_ERR_ALIAS"),
    (dict(beta=fake(9, 4)), "MDN_ERR_ALIGN"),
    (dict(M=None), "MDN_ERR_NULL"),                      # M is required when mu is given
    (dict(mu=None, M=None, v=fake(2, 2)), "MDN_ERR_ALIGN"),   # ... not when mu = 0 (NULL)
    (dict(beta=fake(9), o=fake(9)), "MDN_ERR_ALIAS"),   # output over beta
])
def test_decode_rejects(lib, over, status):
    assert mdn.STATUS_NAMES[call_dec(lib, dec_args(**over))] == status


def test_decode_no_work_returns_ok(lib):
    assert call_dec(lib, dec_args(N=0, q=None)) == 0
    assert call_dec(lib, dec_args(H=0, S=None)) == 0


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        mdn.load_library(str(tmp_path / "libmdn.so"))


def call_prepare(lib, a):
    return lib.mdn_chunk_fwd_prepare(a["q"], a["k"], a["alpha"], a["mu"], a["eta"], a["beta"],
                                     a["B"], a["T"], a["H"], a["Dk"], a["chunk"], a["dt"], a["ws"],
                                     a["wsb"], a["stream"])


def call_scan(lib, a):
    return lib.mdn_chunk_fwd_scan(a["q"], a["k"], a["v"], a["S0"], a["M0"], a["O"], a["S_T"],
                                  a["M_T"], a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["chunk"],
                                  a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(Dk=32), "MDN_ERR_UNSUPPORTED"),
    (dict(T=-1), "MDN_ERR_SHAPE"),
    (dict(k=None), "MDN_ERR_NULL"),
    (dict(alpha=None), "MDN_ERR_NULL"),
    (dict(alpha=fake(3, 4)), "MDN_ERR_ALIGN"),
    (dict(mu=None, k=fake(1, 8)), "MDN_ERR_ALIGN"),   # a NULL mu (mu = 0) passes the NULL check
    (dict(ws=None), "MDN_ERR_WORKSPACE"),
    (dict(ws=fake(1)), "MDN_ERR_ALIAS"),            # workspace over k
    (dict(beta=fake(12, 4)), "MDN_ERR_ALIGN"),
    (dict(beta=fake(12), ws=fake(12)), "MDN_ERR_ALIAS"),   # workspace over beta
])
def test_prepare_rejects(lib, over, status):
    assert mdn.STATUS_NAMES[call_prepare(lib, fwd_args(**over))] == status


def test_prepare_no_work(lib):
    assert call_prepare(lib, fwd_args(T=0, q=None, ws=None)) == 0
    assert call_prepare(lib, fwd_args(B=0, q=None, ws=None)) == 0


@pytest.mark.parametrize("over,status", [
    (dict(Dv=32), "MDN_ERR_UNSUPPORTED"),
    (dict(v=None), "MDN_ERR_NULL"),
    (dict(O=None), "MDN_ERR_NULL"),
    (dict(wsb=64), "MDN_ERR_WORKSPACE"),
    (dict(O=fake(11)), "MDN_ERR_ALIAS"),           # output over the workspace
    (dict(S_T=fake(11, 4096)), "MDN_ERR_ALIAS"),   # final state inside the workspace
    (dict(M_T=fake(6)), "MDN_ERR_ALIAS"),          # final momentum over initial memory
])
def test_scan_rejects(lib, over, status):
    assert mdn.STATUS_NAMES[call_scan(lib, fwd_args(**over))] == status


def gate_args(**over):
    a = dict(ze=fake(0), za=fake(1), zb=fake(2), zm=fake(3), n=1000,
             p=dict(tau=2.0, s=1.0, a=1.0, b=0.0, log_mu_min=-2.0),
             alpha=fake(4), mu=fake(5), eta=fake(6), beta=fake(7), stream=None)
    p = dict(a["p"])
    p.update(over.pop("p", {}))
    a.update(over)
    a["p"] = p
    return a


def call_gates(lib, a):
    return lib.mdn_gates_from_logits(a["ze"], a["za"], a["zb"], a["zm"], a["n"],
                                     mdn.GateParams(**a["p"]), a["alpha"], a["mu"], a["eta"],
                                     a["beta"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(ze=None), "MDN_ERR_NULL"),
    (dict(beta=None), "MDN_ERR_NULL"),
    (dict(za=fake(1, 4)), "MDN_ERR_ALIGN"),
    (dict(mu=fake(5, 8)), "MDN_ERR_ALIGN"),
    (dict(p=dict(tau=0.0)), "MDN_ERR_UNSUPPORTED"),
    (dict(p=dict(tau=-1.0)), "MDN_ERR_UNSUPPORTED"),
    (dict(p=dict(s=float("nan"))), "MDN_ERR_UNSUPPORTED"),
    (dict(p=dict(log_mu_min=float("-inf"))), "MDN_ERR_UNSUPPORTED"),
    (dict(alpha=fake(0)), "MDN_ERR_ALIAS"),              # output over an input
    (dict(eta=fake(5, 1024)), "MDN_ERR_ALIAS"),          # output inside another output
    (dict(n=1 << 62), "MDN_ERR_SHAPE"),
])
def test_gates_rejects(lib, over, status):
    assert mdn.STATUS_NAMES[call_gates(lib, gate_args(**over))] == status


def test_gates_empty_is_ok_and_outputs_never_cover_inputs(lib):
    # n = 0 returns before any pointer is looked at
    assert call_gates(lib, gate_args(n=0, ze=None, alpha=None)) == 0
    # inputs may share one buffer, but an output over it is rejected (a call
    # that passes validation would launch, so only the rejection is checked)
    a = gate_args(za=fake(0), zb=fake(0), zm=fake(0), beta=fake(0, 256))
    assert mdn.STATUS_NAMES[call_gates(lib, a)] == "MDN_ERR_ALIAS"


def call_pro(lib, q=fake(0), k=fake(1), d=None, qo=fake(2), ko=fake(3), rows=10, H=2, D=64,
             eps=1e-6, dt=mdn.MDN_BF16):
    return lib.mdn_qk_prologue(q, k, d, qo, ko, rows, H, D, eps, dt, None)


def call_epi(lib, o=fake(0), g=fake(1), w=None, y=fake(2), rows=10, H=2, D=64, eps=1e-6,
             dt=mdn.MDN_BF16):
    return lib.mdn_output_epilogue(o, g, w, y, rows, H, D, eps, dt, None)


@pytest.mark.parametrize("over,status", [
    (dict(D=96), "MDN_ERR_UNSUPPORTED"),
    (dict(eps=0.0), "MDN_ERR_UNSUPPORTED"),
    (dict(eps=float("nan")), "MDN_ERR_UNSUPPORTED"),
    (dict(dt=7), "MDN_ERR_UNSUPPORTED"),
    (dict(H=-1), "MDN_ERR_SHAPE"),
    (dict(q=None), "MDN_ERR_NULL"),
    (dict(ko=None), "MDN_ERR_NULL"),
    (dict(k=fake(1, 8)), "MDN_ERR_ALIGN"),
    (dict(d=fake(4, 4)), "MDN_ERR_ALIGN"),
    (dict(qo=fake(1)), "MDN_ERR_ALIAS"),            # q_out over k
    (dict(qo=fake(0, 16)), "MDN_ERR_ALIAS"),        # q_out shifted over q, not in place
    (dict(ko=fake(2)), "MDN_ERR_ALIAS"),            # both outputs at one address
])
def test_prologue_rejects(lib, over, status):
    assert mdn.STATUS_NAMES[call_pro(lib, **over)] == status


@pytest.mark.parametrize("over,status", [
    (dict(D=32), "MDN_ERR_UNSUPPORTED"),
    (dict(eps=-1.0), "MDN_ERR_UNSUPPORTED"),
    (dict(o=None), "MDN_ERR_NULL"),
    (dict(w=fake(4, 8)), "MDN_ERR_ALIGN"),
    (dict(y=fake(1)), "MDN_ERR_ALIAS"),             # y over the gate
    (dict(y=fake(0, 32)), "MDN_ERR_ALIAS"),         # y shifted over o
    (dict(rows=1 << 62), "MDN_ERR_SHAPE"),
])
def test_epilogue_rejects(lib, over, status):
    assert mdn.STATUS_NAMES[call_epi(lib, **over)] == status


def test_prologue_epilogue_no_rows(lib):
    assert call_pro(lib, rows=0, q=None) == 0
    assert call_epi(lib, H=0, o=None) == 0


def test_peaks_library_exports_its_header():
    """libmdn_peaks.so (the benchmark's ceiling kernels) exports every
    function include/libmdn_peaks.h declares; its argument checks run on the
    host before any launch."""
    from chunkwise_delta_rule_amd import peaks

    plib = peaks.load_library()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "libmdn_peaks.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(mdn_[a-z0-9_]+)\s*\(", text)))
    assert names == ["mdn_peak_copy", "mdn_peak_mfma_bf16", "mdn_peak_mfma_bf16_flop"]
    for name in names:
        assert ctypes.cast(getattr(plib, name), ctypes.c_void_p).value
    assert plib.mdn_peak_mfma_bf16_flop(3, 5) == 3 * 4 * 5 * 8 * 16 * 16 * 32 * 2
    assert plib.mdn_peak_mfma_bf16_flop(0, 5) == 0
    assert plib.mdn_peak_mfma_bf16(4, 1, None, None) == 1
    assert plib.mdn_peak_mfma_bf16(0, 1, 16, None) == 2
    assert plib.mdn_peak_copy(None, 16, 16, 1, None) == 1
    assert plib.mdn_peak_copy(16, 32, 15, 1, None) == 2
    assert plib.mdn_peak_copy(8, 32, 16, 1, None) == 4
    assert plib.mdn_peak_copy(16, 32, 0, 1, None) == 0


def test_noalloc_validates_before_touching_a_device(lib):
    """mdn_chunk_fwd_noalloc checks its arguments like mdn_chunk_fwd, and a
    problem whose workspace exceeds the library's scratch array is refused
    with MDN_ERR_WORKSPACE, all before any HIP call (fake pointers here)."""
    P = 1 << 20
    ptrs = [P * (i + 1) for i in range(13)]
    call = lambda ptrs, B, T, H, dt: lib.mdn_chunk_fwd_noalloc(*ptrs, B, T, H, 128, 128, 64, dt,
                                                                None)
    B, T, H = 8, 8192, 16
    assert lib.mdn_chunk_fwd_workspace_bytes(B, T, H, 128, 128, 64, mdn.MDN_BF16) > \
        mdn.NOALLOC_SCRATCH_BYTES
    big = [(1 << 40) * (i + 1) for i in range(13)]
    assert call(big, B, T, H, mdn.MDN_BF16) == 6
    assert call(big, B, T, H, mdn.MDN_F32) == 6
    assert call([None] + big[1:], B, T, H, mdn.MDN_BF16) == 1
    assert call(ptrs, -1, T, H, mdn.MDN_BF16) == 2
    assert call(ptrs, 0, T, H, mdn.MDN_BF16) == 0          # nothing to do
    assert lib.mdn_chunk_fwd_noalloc(*ptrs, 1, 64, 1, 96, 128, 64, mdn.MDN_BF16, None) == 3
    assert call([p + 8 for p in ptrs], 1, 64, 1, mdn.MDN_BF16) == 4
