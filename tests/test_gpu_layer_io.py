"""GPU parity of mdn_qk_prologue and mdn_output_epilogue (the elementwise
steps around the core: "MDN: Parallelizing Stepwise Momentum for Delta Linear
Attention" (slides), frame "The memory sits inside a familiar language-model
block"; the reading notes, Sec. 2.9) against the oracle's float64 versions,
element by element.

Tolerance per element, with oracle value r and kernel value x:
  fp32 I/O:  |x - r| <= 1e-5 max|r|   (a few fp32 roundings of O(1) values
             and, in the epilogue, the hardware exponential of the sigmoid)
  bf16 I/O:  |x - r| <= (2^-8 + 4e-6) |r| + 1e-6 max|r|   (one rounding of
             the result to bf16, at most half a bf16 spacing, 2^-8 |r| at the
             bottom of a binade, after fp32 arithmetic that can move a value
             across a rounding boundary by a few 1e-6 of it)
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from chunkwise_delta_rule_amd import mdn

pytestmark = pytest.mark.gpu
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def close(x, r, io, label):
    x = x.float().cpu().numpy().astype(np.float64)
    assert x.shape == r.shape and np.all(np.isfinite(x)), label
    scale = float(np.max(np.abs(r))) if r.size else 0.0
    tol = 1e-5 * scale if io == "f32" else (2.0 ** -8 + 4e-6) * np.abs(r) + 1e-6 * scale
    err = np.abs(x - r)
    worst = float(np.max(err / np.maximum(tol, 1e-300))) if r.size else 0.0
    print(f"  {label}: max|err|={float(np.max(err)) if r.size else 0:.3e} worst err/tol={worst:.3f}")
    assert worst <= 1.0, label


def draw(shape, io, seed, scale=1.0):
    rng = np.random.default_rng(si.SEED_BASE + seed)
    return si.round_io(rng.standard_normal(shape) * scale, io)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rows,H", [(1, 1), (3, 2), (1000, 16), (8 * 4096, 16)])
def test_prologue(io, D, rows, H):
    q = draw((rows, H, D), io, 400 + rows % 97)
    k = draw((rows, H, D), io, 401 + rows % 89)
    d = np.random.default_rng(7).uniform(-0.5, 1.0, H).astype(np.float32)
    for dd in (None, d):
        print(f"prologue {io} D{D} rows{rows} H{H} d={'yes' if dd is not None else 'no'}", flush=True)
        qo, ko = mdn.qk_prologue(torch.from_numpy(q).cuda().to(DT[io]),
                                 torch.from_numpy(k).cuda().to(DT[io]),
                                 None if dd is None else torch.from_numpy(dd).cuda(), eps=1e-6)
        torch.cuda.synchronize()
        rq, rk = oracle.qk_prologue(q, k, dd, eps=float(np.float32(1e-6)))
        close(qo, rq, io, "q_out")
        close(ko, rk, io, "k_out")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rows,H", [(1, 1), (3, 2), (1000, 16), (8 * 4096, 16)])
def test_epilogue(io, D, rows, H):
    o = draw((rows, H, D), io, 410 + rows % 97, scale=0.3)
    g = draw((rows, H, D), io, 411 + rows % 89, scale=2.0)
    w = np.random.default_rng(8).uniform(0.5, 1.5, D).astype(np.float32)
    for ww in (None, w):
        print(f"epilogue {io} D{D} rows{rows} H{H} w={'yes' if ww is not None else 'no'}", flush=True)
        y = mdn.output_epilogue(torch.from_numpy(o).cuda().to(DT[io]),
                                torch.from_numpy(g).cuda().to(DT[io]),
                                None if ww is None else torch.from_numpy(ww).cuda(), eps=1e-6)
        torch.cuda.synchronize()
        close(y, oracle.output_epilogue(o, g, ww, eps=float(np.float32(1e-6))), io, "y")


def test_in_place_and_zero_rows():
    q = draw((50, 4, 128), "bf16", 420)
    k = draw((50, 4, 128), "bf16", 421)
    tq = torch.from_numpy(q).cuda().to(torch.bfloat16)
    tk = torch.from_numpy(k).cuda().to(torch.bfloat16)
    mdn.qk_prologue(tq, tk, out=(tq, tk))
    o = draw((50, 4, 64), "f32", 422)
    to = torch.from_numpy(o).cuda()
    g = torch.zeros_like(to)
    mdn.output_epilogue(to, g, out=to)
    e = torch.empty((0, 4, 64), device="cuda")
    mdn.output_epilogue(e, e)
    mdn.qk_prologue(e, e)
    torch.cuda.synchronize()
    rq, rk = oracle.qk_prologue(q, k, None, eps=float(np.float32(1e-6)))
    close(tq, rq, "bf16", "q in place")
    close(tk, rk, "bf16", "k in place")
    close(to, oracle.output_epilogue(o, np.zeros_like(o), None, eps=float(np.float32(1e-6))),
          "f32", "y in place")
