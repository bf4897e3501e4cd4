"""ctypes binding of libmdn_peaks.so (include/libmdn_peaks.h): the dense bf16
MFMA loop and the streaming copy that give the benchmark measured ceilings
beside the datasheet peaks.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmdn_peaks.so")
_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libmdn_peaks.so not found at {path}; build it first with "
                          "`python -m chunkwise_delta_rule_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.mdn_peak_mfma_bf16_flop.restype = ctypes.c_int64
    lib.mdn_peak_mfma_bf16_flop.argtypes = [I, I]
    lib.mdn_peak_mfma_bf16.restype = I
    lib.mdn_peak_mfma_bf16.argtypes = [I, I, P, P]
    lib.mdn_peak_copy.restype = I
    lib.mdn_peak_copy.argtypes = [P, P, S, I, P]
    if path == LIB_PATH:
        _lib = lib
    return lib


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def mfma_bf16(workgroups: int, iters: int, out: torch.Tensor) -> int:
    """Enqueue one MFMA loop launch; returns its flop.  out: float32 with at
    least workgroups * 256 elements."""
    lib = load_library()
    assert out.dtype == torch.float32 and out.numel() >= workgroups * 256 and out.is_cuda
    st = lib.mdn_peak_mfma_bf16(workgroups, iters, out.data_ptr(), _stream(out.device))
    if st != 0:
        raise RuntimeError(f"mdn_peak_mfma_bf16 failed with status {st}")
    return int(lib.mdn_peak_mfma_bf16_flop(workgroups, iters))


def copy(src: torch.Tensor, dst: torch.Tensor, nontemporal: bool = True) -> int:
    """Enqueue dst <- src (same byte size); returns the bytes moved (read
    plus written)."""
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    assert src.is_cuda and dst.is_cuda and dst.numel() * dst.element_size() == nbytes
    assert src.is_contiguous() and dst.is_contiguous()
    st = lib.mdn_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, int(nontemporal),
                           _stream(src.device))
    if st != 0:
        raise RuntimeError(f"mdn_peak_copy failed with status {st}")
    return 2 * nbytes
