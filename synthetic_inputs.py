"""Seeded synthetic inputs for Momentum DeltaNet forward and decode runs.

This module is shared by the tests, the smoke check and the benchmark, and is
the ONLY code the GPU side and the oracle side have in common.  It draws and
rounds numbers; it holds none of the method's arithmetic.

Recipe (every array is drawn whole, in C order of its layout, from one
``numpy.random.Generator(PCG64(seed))`` in float64):

1. q, k ~ N(0, 1), v ~ N(0, 1), in this order.
2. Gate variates: either three uniform arrays (alpha, mu, eta) or three
   standard-normal arrays z_alpha, z_mu, z_eta mapped as
   alpha = exp(-0.1 softplus(z)), mu = 0.9 sigmoid(z), eta = sigmoid(z).
3. Initial states S0 then M0 when the workload has them.
3b. The update-step gate beta, last, when the workload has one: uniform
   U(0.2, 1) or sigmoid(z) of a standard normal z.  Workloads without it
   draw exactly what they drew before beta existed.
4. q and k are L2-normalised per (token, head) in float64; this mirrors the
   model placing the normalisation in front of the memory core.
5. q, k, v are rounded once to the I/O dtype (round to nearest even);
   gates and states are rounded to float32.

The results are float32 numpy arrays whose values are exactly representable
in the I/O dtype, so the oracle (after exact widening to float64) and the GPU
(after exact narrowing to bf16) see the same numbers.

Shapes: q, k [B, T, H, Dk]; v [B, T, H, Dv]; gates [B, T, H];
states [B, H, Dk, Dv].  Decode: q, k [N, H, Dk]; v [N, H, Dv]; gates [N, H];
states [N, H, Dk, Dv].
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Iterator, Optional

import numpy as np

SEED_BASE = 20260


@dataclass(frozen=True)
class ForwardConfig:
    name: str
    B: int
    T: int
    H: int
    Dk: int
    Dv: int
    chunk: int
    io_dtype: str            # "f32" or "bf16"
    gates: str               # "uniform" or "logit"
    seed: int
    init_state_std: float = 0.0   # 0 => S0 = M0 = 0 (None)
    beta: str = "none"            # "none" (beta = 1, None), "uniform" or "logit"


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    N: int
    H: int
    Dk: int
    Dv: int
    steps: int
    state_std: float
    seed: int
    io_dtype: str = "bf16"
    beta: str = "none"            # as for ForwardConfig


# The workloads: a small fp32 correctness case, a 400M-like layer, the
# 1.3B-like headline layer, a 16K-context layer and the decode loop.
CONFIGS: Dict[int, object] = {
    0: ForwardConfig("fwd-fp32-B1H2T256d64", 1, 256, 2, 64, 64, 64, "f32", "uniform",
                     SEED_BASE + 0),
    1: ForwardConfig("fwd-bf16-B4H8T2048d128", 4, 2048, 8, 128, 128, 64, "bf16", "uniform",
                     SEED_BASE + 1),
    2: ForwardConfig("fwd-bf16-B8H16T4096d128", 8, 4096, 16, 128, 128, 64, "bf16", "logit",
                     SEED_BASE + 2),
    3: ForwardConfig("fwd-bf16-B1H16T16384d128", 1, 16384, 16, 128, 128, 64, "bf16", "logit",
                     SEED_BASE + 3),
    4: DecodeConfig("decode-N256H16d128x512", 256, 16, 128, 128, 512, 0.02, SEED_BASE + 4),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned
    as float32 holding exactly those values.  Rounds straight from float64
    (no intermediate float32 rounding)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    # bfloat16 keeps 7 of float64's 52 fraction bits: round at bit 45
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = (bits + (np.uint64(1) << np.uint64(44)) - np.uint64(1) + lsb) & ~np.uint64(
        (1 << 45) - 1)
    y = rounded.view(np.float64)
    finite = np.isfinite(x)
    big = np.abs(y[finite]) > 3.3895313892515355e38   # largest finite bf16
    tiny = (np.abs(y[finite]) < 1.1754943508222875e-38) & (y[finite] != 0)
    if big.any() or tiny.any():
        raise ValueError("value outside the normal bfloat16 range")
    return y.astype(np.float32)


def round_io(x: np.ndarray, io_dtype: str) -> np.ndarray:
    if io_dtype == "bf16":
        return bf16_round(x)
    if io_dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(io_dtype)


_BLOCK = 1 << 20   # elements per generation block (bounds temporaries)


def _normal_rows(rng: np.random.Generator, shape, io_dtype: str, normalise: bool,
                 scale: float = 1.0) -> np.ndarray:
    """Draw N(0, 1) for a whole array in C order (block by block; the stream
    is the same as one call), optionally L2-normalise each last-axis row in
    float64, scale, and round once to the I/O dtype.  Returns float32."""
    D = shape[-1]
    rows = int(np.prod(shape[:-1]))
    out = np.empty(shape, np.float32)
    flat = out.reshape(rows, D)
    blk = max(1, _BLOCK // D)
    buf = np.empty((min(blk, rows), D))
    for r0 in range(0, rows, blk):
        r1 = min(rows, r0 + blk)
        x = buf[: r1 - r0]
        rng.standard_normal(out=x)
        if normalise:
            x /= np.linalg.norm(x, axis=1, keepdims=True)
        if scale != 1.0:
            x *= scale
        flat[r0:r1] = round_io(x, io_dtype)
    return out


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def _gates(rng: np.random.Generator, shape, kind: str):
    if kind == "uniform":
        a = rng.uniform(0.9, 1.0, size=shape)
        m = rng.uniform(0.0, 0.9, size=shape)
        e = rng.uniform(0.05, 0.5, size=shape)
    elif kind == "logit":
        za = rng.standard_normal(shape)
        zm = rng.standard_normal(shape)
        ze = rng.standard_normal(shape)
        a = np.exp(-0.1 * _softplus(za))
        m = 0.9 * _sigmoid(zm)
        e = _sigmoid(ze)
    else:
        raise ValueError(kind)
    return a.astype(np.float32), m.astype(np.float32), e.astype(np.float32)


def _beta(rng: np.random.Generator, shape, kind: str) -> Optional[np.ndarray]:
    if kind == "none":
        return None
    if kind == "uniform":
        return rng.uniform(0.2, 1.0, size=shape).astype(np.float32)
    if kind == "logit":
        return _sigmoid(rng.standard_normal(shape)).astype(np.float32)
    raise ValueError(kind)


def make_forward(cfg: ForwardConfig, **overrides) -> Dict[str, Optional[np.ndarray]]:
    """Draw one forward workload.  ``overrides`` may replace any field of the
    config (B, T, H, Dk, Dv, seed, init_state_std, ...) to make a smaller or
    different case with the same recipe."""
    if overrides:
        cfg = replace(cfg, **overrides)
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    B, T, H, Dk, Dv = cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv
    q = _normal_rows(rng, (B, T, H, Dk), cfg.io_dtype, normalise=True)
    k = _normal_rows(rng, (B, T, H, Dk), cfg.io_dtype, normalise=True)
    v = _normal_rows(rng, (B, T, H, Dv), cfg.io_dtype, normalise=False)
    alpha, mu, eta = _gates(rng, (B, T, H), cfg.gates)
    S0 = M0 = None
    if cfg.init_state_std > 0:
        S0 = _normal_rows(rng, (B, H, Dk, Dv), "f32", False, cfg.init_state_std)
        M0 = _normal_rows(rng, (B, H, Dk, Dv), "f32", False, cfg.init_state_std)
    beta = _beta(rng, (B, T, H), cfg.beta)
    return dict(q=q, k=k, v=v, alpha=alpha, mu=mu, eta=eta, beta=beta, S0=S0, M0=M0, cfg=cfg)


def decode_initial_state(cfg: DecodeConfig, rng: np.random.Generator):
    shape = (cfg.N, cfg.H, cfg.Dk, cfg.Dv)
    S = _normal_rows(rng, shape, "f32", False, cfg.state_std)
    M = _normal_rows(rng, shape, "f32", False, cfg.state_std)
    return S, M


def decode_token(cfg: DecodeConfig, rng: np.random.Generator) -> Dict[str, np.ndarray]:
    """One decode step's inputs, drawn fresh: q, k L2-normalised, v ~ N(0,1),
    gates from normal logits as in the 1.3B-like layer."""
    N, H = cfg.N, cfg.H
    q = _normal_rows(rng, (N, H, cfg.Dk), cfg.io_dtype, normalise=True)
    k = _normal_rows(rng, (N, H, cfg.Dk), cfg.io_dtype, normalise=True)
    v = _normal_rows(rng, (N, H, cfg.Dv), cfg.io_dtype, normalise=False)
    alpha, mu, eta = _gates(rng, (N, H), "logit")
    beta = _beta(rng, (N, H), cfg.beta)
    return dict(q=q, k=k, v=v, alpha=alpha, mu=mu, eta=eta, beta=beta)


def decode_stream(cfg: DecodeConfig, **overrides) -> Iterator:
    """Yields (S0, M0) first, then one token dict per step."""
    if overrides:
        cfg = replace(cfg, **overrides)
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    yield decode_initial_state(cfg, rng)
    for _ in range(cfg.steps):
        yield decode_token(cfg, rng)


def tokens_per_call(cfg: ForwardConfig) -> int:
    return cfg.B * cfg.T


def gate_logits(n: int, seed: int, scale: float = 3.0) -> Dict[str, np.ndarray]:
    """Four float32 logit arrays of n values each (z_eta, z_alpha, z_beta,
    z_mu, drawn in this order) ~ N(0, scale^2), the first 16 entries of each
    replaced by fixed extremes (+-1e3, +-100, +-30, +-10, +-1, +-1e-3, 0 and
    -0) so that the saturated ends are always covered."""
    rng = np.random.default_rng(SEED_BASE + seed)
    ext = np.array([1e3, -1e3, 100, -100, 30, -30, 10, -10, 1, -1, 1e-3, -1e-3, 0.0, -0.0, 5, -5])
    out = {}
    for name in ("z_eta", "z_alpha", "z_beta", "z_mu"):
        z = rng.normal(0.0, scale, size=n)
        m = min(n, ext.size)
        z[:m] = np.roll(ext, len(out) * 3)[:m]
        out[name] = z.astype(np.float32)
    return out


def backward_cotangents(cfg: ForwardConfig, seed: int, terminal: bool = True,
                        **overrides) -> Dict[str, Optional[np.ndarray]]:
    """Gradients arriving at the forward's outputs, for a backward run on the
    workload ``make_forward(cfg, **overrides)``: dO ~ N(0, 1) rounded to the
    I/O dtype, then (when ``terminal``) dS_T, dM_T ~ N(0, 1) in float32, drawn
    in this order from their own generator (seed ``SEED_BASE + seed``)."""
    if overrides:
        cfg = replace(cfg, **overrides)
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + seed))
    B, T, H, Dk, Dv = cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv
    dO = _normal_rows(rng, (B, T, H, Dv), cfg.io_dtype, normalise=False)
    dS = dM = None
    if terminal:
        dS = _normal_rows(rng, (B, H, Dk, Dv), "f32", False)
        dM = _normal_rows(rng, (B, H, Dk, Dv), "f32", False)
    return dict(dO=dO, dS_T=dS, dM_T=dM)
