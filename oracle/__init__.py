"""fp64 CPU oracle for Momentum DeltaNet -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it and
has no CPU fallback: the oracle exists to check the GPU path, never to stand
in for it.

The arithmetic lives in ``mdn_oracle.c`` (plain C, fp64, OpenMP over heads and
column blocks).  This module only compiles it with the host compiler, loads it
with ctypes and converts arrays to contiguous float64.

Sources:
  [MDN slides]  "MDN: Parallelizing Stepwise Momentum for Delta Linear
                Attention" (slides), Sec. 3.1 Eqs. (3)-(5) for the recurrence;
                Eqs. (7)-(9), (15)-(18), (40)-(42) and the backup frames for
                the chunkwise equations.
  [MDN notes]   reading notes on the same paper, Secs. 2.2-2.6.

The backward pass (``recurrence_backward``) is the reverse-mode derivative of
the recurrence: the pages give its strategy (save the residuals, rebuild the
states; [MDN slides] frame "The implementation trades saved residuals for
throughput", [MDN notes] Sec. 2.6) but no gradient
formulas, so the definition of the derivative is the reference.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mdn_oracle.c")
_LIB = os.path.join(_HERE, "libmdn_oracle.so")

# flags for the checked-against build: no fast-math, so every operation is
# the IEEE double operation the source states
CFLAGS = ["-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"]

_lib = None

# variant flags of the brute-force chunk evaluator (see mdn_oracle.c)
BF_UNSHIFTED_MASK = 1
BF_EQ8_TYPO = 2
BF_EQ10_TYPO = 4


def build(src: str = _SRC, out: str = _LIB, extra: Tuple[str, ...] = ()) -> str:
    """Compile the oracle with gcc.  Returns the path of the shared object."""
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    dp = ctypes.POINTER(ctypes.c_double)
    lib.mdn_oracle_recurrence.restype = ctypes.c_int
    lib.mdn_oracle_recurrence.argtypes = [dp] * 12 + [ctypes.c_int] * 7
    lib.mdn_oracle_recurrence_vt.restype = ctypes.c_int
    lib.mdn_oracle_recurrence_vt.argtypes = [dp] * 13 + [ctypes.c_int] * 7
    lib.mdn_oracle_chunk_bruteforce.restype = ctypes.c_int
    lib.mdn_oracle_chunk_bruteforce.argtypes = [dp] * 12 + [ctypes.c_int] * 8
    lib.mdn_oracle_chunk_gamma.restype = ctypes.c_int
    lib.mdn_oracle_chunk_gamma.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int, dp]
    lib.mdn_oracle_recurrence_backward.restype = ctypes.c_int
    lib.mdn_oracle_recurrence_backward.argtypes = [dp] * 21 + [ctypes.c_int] * 7
    lib.mdn_oracle_max_threads.restype = ctypes.c_int
    lib.mdn_oracle_max_threads.argtypes = []
    return lib


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the oracle library, compiling it first if no build exists."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _f64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x: Optional[np.ndarray]):
    if x is None:
        return ctypes.POINTER(ctypes.c_double)()
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads(lib: Optional[ctypes.CDLL] = None) -> int:
    return int((lib or load()).mdn_oracle_max_threads())


def recurrence(q, k, v, alpha, mu, eta, beta=None, S0=None, M0=None, *,
               col_block: int = 16, nthreads: int = 0, lib: Optional[ctypes.CDLL] = None,
               return_vt: bool = False):
    """Token-by-token MDN recurrence in fp64.

    q, k: [B, T, H, Dk]; v: [B, T, H, Dv]; alpha, mu, eta (, beta): [B, T, H];
    S0, M0: [B, H, Dk, Dv] or None (zero).  Returns (O, S_T, M_T) as float64.
    """
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, mu, eta, beta = _f64(alpha), _f64(mu), _f64(eta), _f64(beta)
    S0, M0 = _f64(S0), _f64(M0)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, T, H, Dv)
    for g in (alpha, mu, eta) + ((beta,) if beta is not None else ()):
        assert g.shape == (B, T, H)
    for s in (S0, M0):
        assert s is None or s.shape == (B, H, Dk, Dv)
    O = np.zeros((B, T, H, Dv))
    ST = np.zeros((B, H, Dk, Dv))
    MT = np.zeros((B, H, Dk, Dv))
    if return_vt:
        VT = np.zeros((B, T, H, Dv))
        rc = lib.mdn_oracle_recurrence_vt(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                          _ptr(mu), _ptr(eta), _ptr(S0), _ptr(M0), _ptr(O),
                                          _ptr(ST), _ptr(MT), _ptr(VT), B, T, H, Dk, Dv,
                                          col_block, nthreads)
        if rc != 0:
            raise RuntimeError(f"mdn_oracle_recurrence_vt failed with code {rc}")
        return O, ST, MT, VT
    rc = lib.mdn_oracle_recurrence(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(mu),
                                   _ptr(eta), _ptr(S0), _ptr(M0), _ptr(O), _ptr(ST), _ptr(MT),
                                   B, T, H, Dk, Dv, col_block, nthreads)
    if rc != 0:
        raise RuntimeError(f"mdn_oracle_recurrence failed with code {rc}")
    return O, ST, MT


def recurrence_backward(q, k, v, alpha, mu, eta, beta=None, S0=None, M0=None, *, dO,
                        dST=None, dMT=None, col_block: int = 16, nthreads: int = 0,
                        lib: Optional[ctypes.CDLL] = None):
    """Reverse-mode derivative of :func:`recurrence` in fp64: the gradients of
    a loss L given dO = dL/dO and dST, dMT = dL/dS_T, dL/dM_T (None: zero).
    Returns a dict with dq, dk, dv, dalpha, dmu, deta, dbeta (None when beta
    is None: beta = 1 is then not an input), dS0 and dM0."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, mu, eta, beta = _f64(alpha), _f64(mu), _f64(eta), _f64(beta)
    S0, M0, dO, dST, dMT = _f64(S0), _f64(M0), _f64(dO), _f64(dST), _f64(dMT)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, T, H, Dv) and dO.shape == v.shape
    for g in (alpha, mu, eta) + ((beta,) if beta is not None else ()):
        assert g.shape == (B, T, H)
    for st in (S0, M0, dST, dMT):
        assert st is None or st.shape == (B, H, Dk, Dv)
    out = dict(dq=np.zeros((B, T, H, Dk)), dk=np.zeros((B, T, H, Dk)),
               dv=np.zeros((B, T, H, Dv)), dalpha=np.zeros((B, T, H)),
               dbeta=None if beta is None else np.zeros((B, T, H)), dmu=np.zeros((B, T, H)),
               deta=np.zeros((B, T, H)), dS0=np.zeros((B, H, Dk, Dv)),
               dM0=np.zeros((B, H, Dk, Dv)))
    rc = lib.mdn_oracle_recurrence_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(mu), _ptr(eta), _ptr(S0),
        _ptr(M0), _ptr(dO), _ptr(dST), _ptr(dMT), _ptr(out["dq"]), _ptr(out["dk"]),
        _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["dbeta"]), _ptr(out["dmu"]),
        _ptr(out["deta"]), _ptr(out["dS0"]), _ptr(out["dM0"]), B, T, H, Dk, Dv, col_block,
        nthreads)
    if rc != 0:
        raise RuntimeError(f"mdn_oracle_recurrence_backward failed with code {rc}")
    return out


def decode_step(q, k, v, alpha, mu, eta, S, M, beta=None, *, nthreads: int = 0,
                lib: Optional[ctypes.CDLL] = None):
    """One recurrent step for N sequences: q, k [N, H, Dk], v [N, H, Dv],
    gates [N, H], S, M [N, H, Dk, Dv].  Returns (o, S_new, M_new).

    This is the recurrence with T = 1: the [N, 1, H, d] token layout is the
    [N, H, d] decode layout.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    g = lambda x: None if x is None else _f64(x).reshape(N, 1, H)
    O, ST, MT = recurrence(q.reshape(N, 1, H, Dk), k.reshape(N, 1, H, Dk),
                           v.reshape(N, 1, H, Dv), g(alpha), g(mu), g(eta), g(beta),
                           S, M, nthreads=nthreads, lib=lib)
    return O.reshape(N, H, Dv), ST, MT


def chunk_bruteforce(q, k, v, alpha, mu, eta, beta=None, S0=None, M0=None, *, chunk: int,
                     gamma_form: int = 0, flags: int = 0, lib: Optional[ctypes.CDLL] = None):
    """Literal fp64 evaluation of the chunkwise equations (tiny inputs only).
    Same arguments and results as :func:`recurrence`, plus the chunk length,
    the statement of gamma to use (0 product-sum, 1 cumulative ratio, 2 log
    domain) and variant flags that switch in flagged erroneous readings."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, mu, eta, beta = _f64(alpha), _f64(mu), _f64(eta), _f64(beta)
    S0, M0 = _f64(S0), _f64(M0)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    O = np.zeros((B, T, H, Dv))
    ST = np.zeros((B, H, Dk, Dv))
    MT = np.zeros((B, H, Dk, Dv))
    rc = lib.mdn_oracle_chunk_bruteforce(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                         _ptr(mu), _ptr(eta), _ptr(S0), _ptr(M0), _ptr(O),
                                         _ptr(ST), _ptr(MT), B, T, H, Dk, Dv, chunk,
                                         gamma_form, flags)
    if rc != 0:
        raise RuntimeError(f"mdn_oracle_chunk_bruteforce failed with code {rc}")
    return O, ST, MT


def chunk_gamma(alpha, mu, beta=None, *, form: int = 0, lib: Optional[ctypes.CDLL] = None):
    """Gamma of one chunk (n = len(alpha)) in the requested form, n x n."""
    lib = lib or load()
    alpha, mu, beta = _f64(alpha), _f64(mu), _f64(beta)
    n = alpha.shape[0]
    G = np.zeros((n, n))
    rc = lib.mdn_oracle_chunk_gamma(_ptr(alpha), _ptr(beta), _ptr(mu), n, form, _ptr(G))
    if rc != 0:
        raise RuntimeError(f"mdn_oracle_chunk_gamma failed with code {rc}")
    return G


def gates_from_logits(z_eta, z_alpha, z_beta, z_mu, *, tau: float, s: float, a: float, b: float,
                      log_mu_min: float):
    """MDN's coupled gate parameterisation in float64, term by term as
    [MDN slides] frame "Coupled gates restrict the spectral region" (the
    paper's Sec. 3.3; [MDN notes] Sec. 2.8) writes it:
        eta = 1 + tanh(z_eta / tau),  theta = arctan(s eta),
        alpha_max = cos^2 theta,  beta_max = sin^2 theta,
        log alpha = f(z_alpha) + log alpha_max,  beta = sigmoid(z_beta) beta_max,
        log mu = max(f(z_mu), log_mu_min),  f(z) = -a softplus(z + b).
    Plain numpy; softplus(x) = log(1 + e^x) as numpy's logaddexp(0, x).
    Returns (alpha, mu, eta, beta)."""
    z = lambda x: np.asarray(x, dtype=np.float64)
    f = lambda x: -a * np.logaddexp(0.0, x + b)
    eta = 1.0 + np.tanh(z(z_eta) / tau)
    theta = np.arctan(s * eta)
    alpha_max = np.cos(theta) ** 2
    beta_max = np.sin(theta) ** 2
    alpha = np.exp(f(z(z_alpha)) + np.log(alpha_max))
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-z(z_beta)))
    beta = sig * beta_max
    mu = np.exp(np.maximum(f(z(z_mu)), log_mu_min))
    return alpha, mu, eta, beta


def qk_prologue(q, k, d=None, *, eps: float):
    """The Comba query correction and L2 normalisation around the core
    ([MDN slides] frame "The memory sits inside a familiar language-model
    block"; [MDN notes] Sec. 2.9), in float64, per token and head over the
    last axis: q' = q - d_h k, q' / sqrt(|q'|^2 + eps), k / sqrt(|k|^2 + eps).
    q, k [..., H, Dk]; d [H] or None."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if d is not None:
        q = q - np.asarray(d, dtype=np.float64)[:, None] * k
    nq = np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
    nk = np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    return q / nq, k / nk


def output_epilogue(o, g, w=None, *, eps: float):
    """The gated output norm before the output projection ([MDN notes]
    Sec. 2.9: y = W_o[sigmoid(W_g x) * RMSNorm(o)]), in float64 per token and
    head over the last axis: sigmoid(g) * o / sqrt(mean(o^2) + eps) * w."""
    o = np.asarray(o, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    y = (1.0 / (1.0 + np.exp(-g))) * (o / rms)
    if w is not None:
        y = y * np.asarray(w, dtype=np.float64)
    return y
