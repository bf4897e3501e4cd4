"""Python binding of libmdn: argument marshalling only.

Every step of the computation runs in libmdn's HIP kernels.  This module
checks devices, dtypes, shapes and contiguity, allocates outputs and the
workspace with torch, and passes raw device pointers plus torch's current
HIP stream through the C ABI declared in ``include/libmdn.h``.  There is no
fallback: if ``libmdn.so`` has not been built, importing the library fails
loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmdn.so")

MDN_F32 = 0
MDN_BF16 = 1
# mdn_fwd_path: how the bf16 forward partitions the carried state
FWD_PATHS = {"auto": 0, "column_tiles": 1, "row_split": 2, "segments": 3}
# MDN_FWD_AUTO runs the row split up to this many tiles of 64 value columns,
# B * H * (Dv / 64) (the rule in api.hip; a CPU test checks the two agree)
ROW_SPLIT_MAX_TILES = 32
CHUNK = 64
NOALLOC_SCRATCH_BYTES = 64 << 20   # MDN_NOALLOC_SCRATCH_BYTES
HEAD_DIMS = (64, 128)

STATUS_NAMES = {
    0: "MDN_OK",
    1: "MDN_ERR_NULL",
    2: "MDN_ERR_SHAPE",
    3: "MDN_ERR_UNSUPPORTED",
    4: "MDN_ERR_ALIGN",
    5: "MDN_ERR_ALIAS",
    6: "MDN_ERR_WORKSPACE",
    7: "MDN_ERR_HIP",
}

# every symbol include/libmdn.h declares
EXPORTED = ("mdn_set_fwd_path", "mdn_fwd_segment_count", "mdn_chunk_fwd_workspace_bytes",
            "mdn_chunk_fwd_split_workspace_bytes", "mdn_chunk_fwd", "mdn_chunk_fwd_noalloc",
            "mdn_chunk_fwd_prepare", "mdn_chunk_fwd_scan", "mdn_decode_step",
            "mdn_gates_from_logits", "mdn_chunk_bwd_workspace_bytes", "mdn_chunk_bwd",
            "mdn_qk_prologue", "mdn_output_epilogue", "mdn_status_string")


class GateParams(ctypes.Structure):
    """mdn_gate_params, passed by value: f(z) = -a softplus(z + b)."""
    _fields_ = [("tau", ctypes.c_float), ("s", ctypes.c_float), ("a", ctypes.c_float),
                ("b", ctypes.c_float), ("log_mu_min", ctypes.c_float)]


class MdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmdn.so (built in-tree by ``chunkwise_delta_rule_amd.build``)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libmdn.so not found at {path}; build it first with "
                          "`python -m chunkwise_delta_rule_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.mdn_set_fwd_path.restype = I
    lib.mdn_set_fwd_path.argtypes = [I]
    lib.mdn_fwd_segment_count.restype = I
    lib.mdn_fwd_segment_count.argtypes = [I] * 6
    lib.mdn_chunk_fwd_workspace_bytes.restype = S
    lib.mdn_chunk_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.mdn_chunk_fwd_split_workspace_bytes.restype = S
    lib.mdn_chunk_fwd_split_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.mdn_chunk_fwd.restype = I
    lib.mdn_chunk_fwd.argtypes = [P] * 13 + [I] * 7 + [P, S, P]
    lib.mdn_chunk_fwd_noalloc.restype = I
    lib.mdn_chunk_fwd_noalloc.argtypes = [P] * 13 + [I] * 7 + [P]
    lib.mdn_chunk_fwd_prepare.restype = I
    lib.mdn_chunk_fwd_prepare.argtypes = [P] * 6 + [I] * 6 + [P, S, P]
    lib.mdn_chunk_fwd_scan.restype = I
    lib.mdn_chunk_fwd_scan.argtypes = [P] * 8 + [I] * 7 + [P, S, P]
    lib.mdn_decode_step.restype = I
    lib.mdn_decode_step.argtypes = [P] * 10 + [I] * 5 + [P]
    lib.mdn_chunk_bwd_workspace_bytes.restype = S
    lib.mdn_chunk_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.mdn_chunk_bwd.restype = I
    lib.mdn_chunk_bwd.argtypes = [P] * 22 + [I] * 7 + [P, S, P]
    F = ctypes.c_float
    lib.mdn_qk_prologue.restype = I
    lib.mdn_qk_prologue.argtypes = [P] * 5 + [S, I, I, F, I, P]
    lib.mdn_output_epilogue.restype = I
    lib.mdn_output_epilogue.argtypes = [P] * 4 + [S, I, I, F, I, P]
    lib.mdn_gates_from_logits.restype = I
    lib.mdn_gates_from_logits.argtypes = [P] * 4 + [S, GateParams] + [P] * 4 + [P]
    lib.mdn_status_string.restype = ctypes.c_char_p
    lib.mdn_status_string.argtypes = [I]
    if path == LIB_PATH:
        _lib = lib
    return lib


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MDN_BF16
    if t == torch.float32:
        return MDN_F32
    raise TypeError(f"q, k, v must be bfloat16 or float32, got {t}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None or t.numel() == 0:
        return None
    return t.data_ptr()


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def set_fwd_path(path: str) -> str:
    """Select the bf16 forward's state partition for every later call
    (mdn_set_fwd_path): "auto", "column_tiles", "row_split" or "segments".
    Returns the previous setting's name."""
    if path not in FWD_PATHS:
        raise ValueError(f"unknown forward path {path!r}; one of {sorted(FWD_PATHS)}")
    prev = load_library().mdn_set_fwd_path(FWD_PATHS[path])
    return {v: k for k, v in FWD_PATHS.items()}[prev]


def segment_count(B: int, T: int, H: int, Dk: int, Dv: int, with_mu: bool) -> int:
    """Segments a bf16 forward of this shape runs the segment scan with under
    the current forward path, 0 when it runs another path
    (mdn_fwd_segment_count)."""
    return load_library().mdn_fwd_segment_count(B, T, H, Dk, Dv, int(bool(with_mu)))


class fwd_path:
    """Context manager: run the enclosed calls with one forward path."""

    def __init__(self, path: str):
        self.path = path
        self.prev = None

    def __enter__(self):
        self.prev = set_fwd_path(self.path)
        return self

    def __exit__(self, *exc):
        set_fwd_path(self.prev)
        return False


def workspace_bytes(B: int, T: int, H: int, Dk: int, Dv: int, dtype: torch.dtype,
                    chunk: int = CHUNK, split: bool = False) -> int:
    """Workspace bytes of mdn_chunk_fwd (split=False) or of the
    mdn_chunk_fwd_prepare / mdn_chunk_fwd_scan pair (split=True)."""
    lib = load_library()
    fn = lib.mdn_chunk_fwd_split_workspace_bytes if split else lib.mdn_chunk_fwd_workspace_bytes
    return int(fn(B, T, H, Dk, Dv, chunk, _dtype_code(dtype)))


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
              mu: torch.Tensor, eta: torch.Tensor, S0: Optional[torch.Tensor] = None,
              M0: Optional[torch.Tensor] = None, *, beta: Optional[torch.Tensor] = None,
              chunk: int = CHUNK, O: Optional[torch.Tensor] = None,
              S_T: Optional[torch.Tensor] = None, M_T: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, final_state: bool = True,
              Vt: Optional[torch.Tensor] = None, noalloc: bool = False
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Chunkwise MDN forward.  q, k [B, T, H, Dk], v [B, T, H, Dv] (bf16 or
    fp32), gates [B, T, H] fp32 (beta optional: None means beta = 1; mu may
    be None, meaning mu = 0, the gated delta rule), S0/M0 [B, H, Dk, Dv] fp32
    or None.  Vt, when given ([B, T, H, Dv], q's dtype), receives every
    token's residual (the activations mdn_chunk_bwd can take instead of
    recomputing them).
    Returns (O, S_T, M_T); S_T/M_T are None when ``final_state`` is False and
    none were passed in.  ``noalloc`` calls mdn_chunk_fwd_noalloc, which runs
    on the library's own per-device scratch array instead of a workspace (the
    outputs are still allocated here unless passed in)."""
    lib = load_library()
    dev = q.device
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(dt)
    _check(q, "q", (B, T, H, Dk), dt, dev)
    _check(k, "k", (B, T, H, Dk), dt, dev)
    _check(v, "v", (B, T, H, Dv), dt, dev)
    for name, g in (("alpha", alpha), ("mu", mu), ("eta", eta), ("beta", beta)):
        if g is not None or name in ("alpha", "eta"):
            _check(g, name, (B, T, H), torch.float32, dev)
    for name, s in (("S0", S0), ("M0", M0)):
        if s is not None:
            _check(s, name, (B, H, Dk, Dv), torch.float32, dev)
    if O is None:
        O = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    _check(O, "O", (B, T, H, Dv), dt, dev)
    if Vt is not None:
        _check(Vt, "Vt", (B, T, H, Dv), dt, dev)
    if final_state and S_T is None:
        S_T = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    if final_state and M_T is None:
        M_T = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    for name, s in (("S_T", S_T), ("M_T", M_T)):
        if s is not None:
            _check(s, name, (B, H, Dk, Dv), torch.float32, dev)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc runs on the library's own scratch array; pass no workspace")
        st = lib.mdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(mu),
                                       _ptr(eta), _ptr(beta), _ptr(S0), _ptr(M0), _ptr(O),
                                       _ptr(Vt), _ptr(S_T), _ptr(M_T), B, T, H, Dk, Dv, chunk,
                                       code, _stream(dev))
        if st != 0:
            raise MdnError(st, "mdn_chunk_fwd_noalloc")
        return O, S_T, M_T
    need = int(lib.mdn_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, chunk, code))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.mdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(mu), _ptr(eta),
                           _ptr(beta), _ptr(S0), _ptr(M0), _ptr(O), _ptr(Vt), _ptr(S_T),
                           _ptr(M_T), B, T, H, Dk, Dv, chunk, code, _ptr(workspace), wbytes,
                           _stream(dev))
    if st != 0:
        raise MdnError(st, "mdn_chunk_fwd")
    return O, S_T, M_T


class ChunkPlan:
    """Pre-validated arguments for repeated forward calls on fixed buffers:
    the phases can then be launched (and timed) one by one.  Holds the
    outputs and the workspace; launching performs no allocation."""

    def __init__(self, q, k, v, alpha, mu, eta, S0=None, M0=None, *, beta=None,
                 chunk: int = CHUNK, final_state: bool = True, save_vt: bool = False):
        self.lib = load_library()
        self.args = (q, k, v, alpha, mu, eta, S0, M0)
        self.beta = beta
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        self.shape = (B, T, H, Dk, Dv)
        self.chunk = chunk
        self.code = _dtype_code(q.dtype)
        dev = q.device
        self.O = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev)
        self.Vt = torch.empty((B, T, H, Dv), dtype=q.dtype, device=dev) if save_vt else None
        self.S_T = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) if final_state else None
        self.M_T = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) if final_state else None
        # room for the two phases and for a whole call under the current
        # forward path (the segment scan's can be the larger)
        need = max(int(self.lib.mdn_chunk_fwd_split_workspace_bytes(B, T, H, Dk, Dv, chunk,
                                                                    self.code)),
                   int(self.lib.mdn_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, chunk, self.code)))
        self.workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        self.ws_bytes = need
        # one full call validates every argument (and fills the outputs)
        chunk_fwd(*self.args, beta=beta, chunk=chunk, O=self.O, S_T=self.S_T, M_T=self.M_T,
                  workspace=self.workspace, Vt=self.Vt)
        self.stream = _stream(dev)

    def prepare(self):
        q, k, _, a, m, e, _, _ = self.args
        B, T, H, Dk, _ = self.shape
        st = self.lib.mdn_chunk_fwd_prepare(_ptr(q), _ptr(k), _ptr(a), _ptr(m), _ptr(e),
                                            _ptr(self.beta), B, T, H, Dk, self.chunk, self.code,
                                            _ptr(self.workspace), self.ws_bytes, self.stream)
        if st != 0:
            raise MdnError(st, "mdn_chunk_fwd_prepare")

    def scan(self):
        q, k, v, _, _, _, S0, M0 = self.args
        B, T, H, Dk, Dv = self.shape
        st = self.lib.mdn_chunk_fwd_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(S0), _ptr(M0),
                                         _ptr(self.O), _ptr(self.S_T), _ptr(self.M_T), B, T, H,
                                         Dk, Dv, self.chunk, self.code, _ptr(self.workspace),
                                         self.ws_bytes, self.stream)
        if st != 0:
            raise MdnError(st, "mdn_chunk_fwd_scan")

    def forward(self):
        q, k, v, a, m, e, S0, M0 = self.args
        B, T, H, Dk, Dv = self.shape
        st = self.lib.mdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(m), _ptr(e),
                                    _ptr(self.beta), _ptr(S0), _ptr(M0), _ptr(self.O),
                                    _ptr(self.Vt), _ptr(self.S_T),
                                    _ptr(self.M_T), B, T, H, Dk, Dv, self.chunk, self.code,
                                    _ptr(self.workspace), self.ws_bytes, self.stream)
        if st != 0:
            raise MdnError(st, "mdn_chunk_fwd")


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                mu: Optional[torch.Tensor], eta: torch.Tensor, S: torch.Tensor,
                M: Optional[torch.Tensor], o: Optional[torch.Tensor] = None, *,
                beta: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step: q, k [N, H, Dk], v [N, H, Dv], gates [N, H] (beta
    optional: None means beta = 1; mu None means mu = 0, and then M may be
    None); S, M [N, H, Dk, Dv] fp32 updated in place.  Returns o [N, H, Dv]."""
    lib = load_library()
    dev = q.device
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(dt)
    _check(q, "q", (N, H, Dk), dt, dev)
    _check(k, "k", (N, H, Dk), dt, dev)
    _check(v, "v", (N, H, Dv), dt, dev)
    for name, g in (("alpha", alpha), ("mu", mu), ("eta", eta), ("beta", beta)):
        if g is not None or name in ("alpha", "eta"):
            _check(g, name, (N, H), torch.float32, dev)
    _check(S, "S", (N, H, Dk, Dv), torch.float32, dev)
    if M is not None or mu is not None:
        _check(M, "M", (N, H, Dk, Dv), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, Dv), dtype=dt, device=dev)
    _check(o, "o", (N, H, Dv), dt, dev)
    st = lib.mdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(mu), _ptr(eta),
                             _ptr(beta), _ptr(S), _ptr(M), _ptr(o), N, H, Dk, Dv, code,
                             _stream(dev))
    if st != 0:
        raise MdnError(st, "mdn_decode_step")
    return o


def gates_from_logits(z_eta: torch.Tensor, z_alpha: torch.Tensor, z_beta: torch.Tensor,
                      z_mu: torch.Tensor, *, tau: float, s: float, a: float, b: float,
                      log_mu_min: float = -2.0,
                      out: Optional[Tuple[torch.Tensor, ...]] = None
                      ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """MDN's coupled gates from logits (float32, one shape for all four, e.g.
    [B, T, H]).  Returns (alpha, mu, eta, beta) of that shape, float32, in
    the form chunk_fwd and decode_step take them."""
    lib = load_library()
    dev = z_eta.device
    shape = tuple(z_eta.shape)
    for name, z in (("z_eta", z_eta), ("z_alpha", z_alpha), ("z_beta", z_beta), ("z_mu", z_mu)):
        _check(z, name, shape, torch.float32, dev)
    if out is None:
        out = tuple(torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(4))
    for name, g in zip(("alpha", "mu", "eta", "beta"), out):
        _check(g, name, shape, torch.float32, dev)
    n = z_eta.numel()
    p = GateParams(tau, s, a, b, log_mu_min)
    st = lib.mdn_gates_from_logits(_ptr(z_eta), _ptr(z_alpha), _ptr(z_beta), _ptr(z_mu), n, p,
                                   *(_ptr(g) for g in out), _stream(dev))
    if st != 0:
        raise MdnError(st, "mdn_gates_from_logits")
    return tuple(out)


def workspace_bytes_bwd(B: int, T: int, H: int, Dk: int, Dv: int, dtype: torch.dtype,
                        chunk: int = CHUNK) -> int:
    """Workspace bytes of mdn_chunk_bwd."""
    return int(load_library().mdn_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk,
                                                            _dtype_code(dtype)))


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
              mu: Optional[torch.Tensor], eta: torch.Tensor, S0: Optional[torch.Tensor],
              M0: Optional[torch.Tensor], dO: torch.Tensor, dS_T: Optional[torch.Tensor] = None,
              dM_T: Optional[torch.Tensor] = None, *, beta: Optional[torch.Tensor] = None,
              chunk: int = CHUNK, workspace: Optional[torch.Tensor] = None,
              state_grads: bool = True, Vt: Optional[torch.Tensor] = None) -> dict:
    """Gradients through mdn_chunk_fwd given dO (and optionally dS_T, dM_T).
    Arguments as for chunk_fwd; returns a dict of float32 tensors dq, dk, dv,
    dalpha, dmu (None without mu), deta, dbeta (None without beta), dS0, dM0
    (None when state_grads is False).  Vt: the residuals chunk_fwd saved for
    these inputs (the states are then rebuilt without the solve)."""
    lib = load_library()
    dev = q.device
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    code = _dtype_code(dt)
    _check(q, "q", (B, T, H, Dk), dt, dev)
    _check(k, "k", (B, T, H, Dk), dt, dev)
    _check(v, "v", (B, T, H, Dv), dt, dev)
    _check(dO, "dO", (B, T, H, Dv), dt, dev)
    if Vt is not None:
        _check(Vt, "Vt", (B, T, H, Dv), dt, dev)
    for name, g in (("alpha", alpha), ("mu", mu), ("eta", eta), ("beta", beta)):
        if g is not None or name in ("alpha", "eta"):
            _check(g, name, (B, T, H), torch.float32, dev)
    for name, st in (("S0", S0), ("M0", M0), ("dS_T", dS_T), ("dM_T", dM_T)):
        if st is not None:
            _check(st, name, (B, H, Dk, Dv), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, T, H, Dk), **f32), dk=torch.empty((B, T, H, Dk), **f32),
               dv=torch.empty((B, T, H, Dv), **f32), dalpha=torch.empty((B, T, H), **f32),
               dmu=torch.empty((B, T, H), **f32) if mu is not None else None,
               deta=torch.empty((B, T, H), **f32),
               dbeta=torch.empty((B, T, H), **f32) if beta is not None else None,
               dS0=torch.empty((B, H, Dk, Dv), **f32) if state_grads else None,
               dM0=torch.empty((B, H, Dk, Dv), **f32) if state_grads else None)
    need = int(lib.mdn_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk, code))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = lib.mdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(mu), _ptr(eta),
                           _ptr(beta), _ptr(S0), _ptr(M0), _ptr(dO), _ptr(dS_T), _ptr(dM_T),
                           _ptr(Vt),
                           *(_ptr(out[n]) for n in ("dq", "dk", "dv", "dalpha", "dmu", "deta",
                                                    "dbeta", "dS0", "dM0")),
                           B, T, H, Dk, Dv, chunk, code, _ptr(workspace), workspace.numel(),
                           _stream(dev))
    if st != 0:
        raise MdnError(st, "mdn_chunk_bwd")
    return out


def qk_prologue(q: torch.Tensor, k: torch.Tensor, d: Optional[torch.Tensor] = None, *,
                eps: float = 1e-6, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
                ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Comba correction q - d_h k and L2 normalisation of q and k (per token
    and head).  q, k [..., H, Dk] contiguous, one dtype; d [H] float32 or
    None.  Returns (q_out, k_out); pass out=(q, k) to work in place."""
    lib = load_library()
    dev = q.device
    shape = tuple(q.shape)
    H, Dk = shape[-2], shape[-1]
    rows = q.numel() // (H * Dk) if q.numel() else 0
    _check(q, "q", shape, q.dtype, dev)
    _check(k, "k", shape, q.dtype, dev)
    if d is not None:
        _check(d, "d", (H,), torch.float32, dev)
    qo, ko = out if out is not None else (torch.empty_like(q), torch.empty_like(k))
    _check(qo, "q_out", shape, q.dtype, dev)
    _check(ko, "k_out", shape, q.dtype, dev)
    st = lib.mdn_qk_prologue(_ptr(q), _ptr(k), _ptr(d), _ptr(qo), _ptr(ko), rows, H, Dk, eps,
                             _dtype_code(q.dtype), _stream(dev))
    if st != 0:
        raise MdnError(st, "mdn_qk_prologue")
    return qo, ko


def output_epilogue(o: torch.Tensor, g: torch.Tensor, w: Optional[torch.Tensor] = None, *,
                    eps: float = 1e-6, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = sigmoid(g) * RMSNorm(o) * w per token and head over Dv.  o, g
    [..., H, Dv] contiguous, one dtype; w [Dv] float32 or None."""
    lib = load_library()
    dev = o.device
    shape = tuple(o.shape)
    H, Dv = shape[-2], shape[-1]
    rows = o.numel() // (H * Dv) if o.numel() else 0
    _check(o, "o", shape, o.dtype, dev)
    _check(g, "g", shape, o.dtype, dev)
    if w is not None:
        _check(w, "w", (Dv,), torch.float32, dev)
    y = out if out is not None else torch.empty_like(o)
    _check(y, "y", shape, o.dtype, dev)
    st = lib.mdn_output_epilogue(_ptr(o), _ptr(g), _ptr(w), _ptr(y), rows, H, Dv, eps,
                                 _dtype_code(o.dtype), _stream(dev))
    if st != 0:
        raise MdnError(st, "mdn_output_epilogue")
    return y
