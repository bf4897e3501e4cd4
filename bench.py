"""Benchmark of the MDN hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--settle SEC] [--decode-steps D] [--no-cpu-baseline]
                    [--no-backward] [--no-decode] [--no-sweep] [--no-configs] [--no-peaks]

A step is one chunkwise forward (mdn_chunk_fwd: coefficients, Gram products,
residual solve, outputs and carried state, one fused kernel for bf16) over
the 1.3B-like layer B=8, H=16,
T=4096, d_k=d_v=128, chunk 64, bf16 q/k/v with fp32 gates and state, inputs
resident in HBM.  `value` is tokens/s = B*T per step / time per step.
Each timed section is preceded by about SEC seconds of untimed calls (the
GPU clock leaves its idle state) and W warm-up steps; then K steps are timed.

The same JSON line carries:
  roofline      the step's kernel against the roof its algorithmic work reaches
                last: bytes it must move vs the HBM peak, or FLOP vs the bf16 MFMA
                peak; timed with HIP events on the launch stream; `traffic` is its
                counter-measured HBM bytes per launch (null once its sources differ
                from the profiled ones);
  kernels       the same record for every kernel of the step;
  split_path    the same forward through mdn_chunk_fwd_prepare + mdn_chunk_fwd_scan;
  forward.from_logits  mdn_gates_from_logits, then the four-gate forward on its gates;
  forward.with_prologue_epilogue  mdn_qk_prologue, the forward, mdn_output_epilogue;
  forward       the whole step against both roofs;
  backward      mdn_chunk_bwd on the same layer (all gradients), against the matrix
                peak of its mix (bf16 products at the bf16 peak, the rest at fp32's);
  decode        the recurrent decode step at 256 sequences x 16 heads, d 128
                (GB/s of algorithmic state + token traffic);
  timing_ab     the headline call timed one call at a time: median of 20 back to
                back, and median of 20 with a 1 GiB write between calls;
  other_configs the 400M-like layer (B4 H8 T2048) and the 16K-context layer
                (B1 H16 T16384) as drawn and with no mu, each under the partitions
                of the state (column tiles, row split, segment scan) with its
                roofline, and the one the default rule runs;
  sweep         tokens/s at T x B = 16384 tokens per call for T = 2K .. 16K;
  measured_peaks  a dense bf16 MFMA loop and a 2 GiB streaming copy on this GPU,
                beside the datasheet peaks;
  cpu_baseline  the fp64 oracle timed on this host's cores.
Rank 0 prints one JSON line; only one GPU is supported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MDN chunkwise fwd tokens/s at H=16,d=128,T=4096; % MFMA peak; decode GB/s"
PEAK_BF16_FLOPS = 2.5e15        # MI355X dense bf16 MFMA
PEAK_HBM_BPS = 8.0e12           # MI355X HBM3E

# algorithmic work (dense count, d = d_k = d_v, C = 64), per token and head
D, C = 128, 64
FLOP_SCAN = 12 * D * D + 4 * C * D       # K[S|M], Q[S|M], K^T[Vt], T R, A Vt
FLOP_PREP = 4 * C * D                    # K K^T, Q K^T
FLOP_FWD = FLOP_SCAN + FLOP_PREP         # 12 d^2 + 8 C d
BYTES_FWD = 3 * D * 2 + D * 2 + 3 * 4    # q, k, v, O (bf16) + three gates (fp32)
BYTES_FWD_BETA = BYTES_FWD + 4            # ... + the optional update-step gate beta
# per kernel, per token and head: what each phase must read and write once
BYTES_TA = 2 * C * C * 2 // C            # T and A, two C x C bf16 matrices per C tokens
BYTES_VEC = 6 * 4                        # six coefficient rows (fp32) the scan reads
BYTES_SCAN = 3 * D * 2 + D * 2 + BYTES_TA + BYTES_VEC     # + final S, M per (b, h)
BYTES_PREP = 2 * D * 2 + 3 * 4 + BYTES_TA + BYTES_VEC
STATE_BYTES_HEAD = 2 * D * D * 4         # S_T and M_T written once per (b, h)
DEC_BYTES_HEAD = 4 * D * D * 4 + 3 * D * 2 + D * 2 + 3 * 4   # S, M in+out; q k v o; gates
DEC_BYTES_HEAD_GDN = 2 * D * D * 4 + 3 * D * 2 + D * 2 + 2 * 4   # mu = 0: S only; two gates
BYTES_GATES = 4 * 4 + 4 * 4              # four fp32 logits in, four fp32 gates out
BYTES_PROLOGUE = 2 * D * 2 + 2 * D * 2   # q, k in and out (bf16)
BYTES_EPILOGUE = 2 * D * 2 + D * 2       # o, gate in, y out (bf16)
# backward (mdn_chunk_bwd), dense products per token and head: prepare 4 C d; reverse scan
# 12 d^2 + 4 C d; re-scan 8 d^2 + 2 C d; per-chunk gradients 12 d^2 + 16 C d
FLOP_BWD = 32 * D * D + 26 * C * D
# what it must read and write once: q, k, v, dO (bf16), three gates in, dq, dk, dv (fp32)
# and three gate gradients out, plus S0, M0 read / dS0, dM0 written per (b, h) (zero here)
BYTES_BWD = 4 * D * 2 + 3 * 4 + 3 * D * 4 + 3 * 4
# with the forward's saved residuals the re-scan only rebuilds the states (4 d^2 instead of
# 8 d^2 + 2 C d) and reads Vt (bf16) instead of v
FLOP_BWD_SAVED = FLOP_BWD - 4 * D * D - 2 * C * D
BYTES_BWD_SAVED = BYTES_BWD + D * 2
PEAK_FP32_MFMA = 157.3e12       # MI355X dense fp32 matrix
# for bf16 I/O these run on bf16 MFMA: the reverse scan's products (12 d^2 + 4 C d), the
# re-scan's (8 d^2 + 2 C d; 4 d^2 with saved residuals), the per-chunk kernel's six state
# products (12 d^2) and its chunk products dO Vt^T, K K^T, Q K^T (6 C d); the rest (prepare,
# the chunk product dR Vt^T and the masked products, 14 C d) is fp32
FLOP_BWD_BF16 = 32 * D * D + 12 * C * D
FLOP_BWD_BF16_SAVED = 28 * D * D + 10 * C * D


def mixed_peak(flop, flop_bf16):
    """The matrix peak of a mix: all flop at their own type's dense peak, in
    the time that takes."""
    return flop / (flop_bf16 / PEAK_BF16_FLOPS + (flop - flop_bf16) / PEAK_FP32_MFMA)
GATE_TAU = (2048 / 16) ** 0.5            # the temperature sqrt(d_in / h) at d_in 2048, 16 heads

# HBM traffic per launch from rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, KiB per dispatch,
# means over the profiled dispatches), recorded with the kernel sources whose sha256 is given;
# the factors scale each counter to bytes as measured on torch's fp32 -> bf16 copy of
# 67,108,864 elements (reads 262,144 KiB, FETCH_SIZE 131,093.9; writes 131,072 KiB, WRITE_SIZE
# 131,072.0).  An entry that covers several kernels of one call sums their dispatches.
# Figures and commands: profiles/chunk_fwd_fused_B8H16T4096d128.md,
# profiles/chunk_fwd_split_B8H16T4096d128.md, profiles/decode_step_N256H16d128.md and
# profiles/gates_from_logits_B8H16T4096.md, profiles/chunk_bwd_B8H16T4096d128.md and
# profiles/layer_prologue_epilogue_B8H16T4096d128.md.
# A kernel whose sources changed reports traffic null.
FETCH_FACTOR = 262144.0 / 131093.9
WRITE_FACTOR = 131072.0 / 131072.0
CSRC = os.path.join(ROOT, "chunkwise_delta_rule_amd", "csrc")
_SPLIT_SHA = "4c566b0ae7c2d13b3231f4104da8130aabf3c8d4d6bdd74f3a0e879a52ee8e85"
_BWD_SHA = "69e0712028edb127a8a18ce0511732f031077c24d0119ba9b3e8389faf6a4536"
_FUSED_SHA = "24ac34770bdef1e6240a3e3c8c87a37fd6ff035907f6b59407384dc8f95348b7"
_LIO_SHA = "627a8009335ec269a3313bb348dbbb8e2230dded01b1dfc19a85d20d78a2a663"
TRAFFIC = {
    # chunk_coef_kernel (3,211.4 / 51,459.6) + chunk_fwd_fused_kernel (223,501.4 / 147,456.2):
    # one mdn_chunk_fwd call, the unit the bench times
    "chunk_fwd_fused_kernel": dict(sources=("chunk_fused.hip", "chunk_common.hpp", "mfma.hpp"),
                                   fetch_kib=3211.4 + 223501.4, write_kib=51459.6 + 147456.2,
                                   sha256=_FUSED_SHA),
    "chunk_scan_bf16_kernel": dict(sources=("chunk_fwd.hip", "chunk_common.hpp", "mfma.hpp"),
                                   fetch_kib=268387.0, write_kib=147457.6, sha256=_SPLIT_SHA),
    "chunk_prep_kernel": dict(sources=("chunk_fwd.hip", "chunk_common.hpp", "mfma.hpp"),
                              fetch_kib=134327.7, write_kib=143909.4, sha256=_SPLIT_SHA),
    # the other configurations' calls under the partition the default rule picks: the
    # 400M-like layer (B4 H8 T2048) on the column tiles, chunk_coef_kernel (421.0 / 6,432.0)
    # + chunk_fwd_fused_kernel (28,173.0 / 20,480.0); the 16K-context layer (B1 H16 T16384)
    # on the segment scan (4 segments): chunk_coef_kernel (1,573.0 / 25,728.3), pass 1 of
    # chunk_fwd_seg_kernel (69,028.2 / 26,880.0), seg_combine_kernel (7,215.0 / 4,096.0) and
    # pass 2 (93,609.3 / 55,040.0); with mu = 0 (5 segments): 1,061.0 / 25,728.3,
    # 66,819.1 / 15,872.0, 3,618.0 / 3,072.0, 99,119.9 / 58,880.0
    "config1_fused": dict(sources=("chunk_fused.hip", "chunk_common.hpp", "mfma.hpp"),
                          fetch_kib=421.0 + 28173.0, write_kib=6432.0 + 20480.0,
                          sha256=_FUSED_SHA),
    "config3_segments": dict(sources=("chunk_fused.hip", "chunk_common.hpp", "mfma.hpp"),
                             fetch_kib=1573.0 + 69028.2 + 7215.0 + 93609.3,
                             write_kib=25728.3 + 26880.0 + 4096.0 + 55040.0, sha256=_FUSED_SHA),
    "config3_segments_no_mu": dict(sources=("chunk_fused.hip", "chunk_common.hpp", "mfma.hpp"),
                                   fetch_kib=1061.0 + 66819.1 + 3618.0 + 99119.9,
                                   write_kib=25728.3 + 15872.0 + 3072.0 + 58880.0,
                                   sha256=_FUSED_SHA),
    "decode_step_kernel": dict(sources=("decode.hip", "mfma.hpp"), fetch_kib=264109.0,
                               write_kib=525524.5, sha256="8fa39113008b99235e1abe57028f0d81"
                               "9b837f475aa87000a6b4e46e3ea6c4e5"),
    # one mdn_chunk_bwd call with the forward's saved residuals: chunk_prep_kernel
    # (134,327.7 / 143,909.4) + bwd_scan_bf16_kernel (268,439.2 / 786,490.1) +
    # bwd_rescan_bf16_kernel with saved residuals (137,299.6 / 524,288.6) +
    # bwd_grad_bf16_kernel<..., true> (929,570.3 / 544,532.0)
    "chunk_bwd": dict(sources=("chunk_bwd.hip", "chunk_fwd.hip", "chunk_common.hpp", "mfma.hpp"),
                      fetch_kib=134327.7 + 268439.2 + 137299.6 + 929570.3,
                      write_kib=143909.4 + 786490.1 + 524288.6 + 544532.0, sha256=_BWD_SHA),
    # the same recomputing the residuals: bwd_rescan_bf16_kernel (170,149.6 / 786,461.9),
    # bwd_grad_bf16_kernel<..., false> (994,744.1 / 542,284.8)
    "chunk_bwd_recompute": dict(sources=("chunk_bwd.hip", "chunk_fwd.hip", "chunk_common.hpp",
                                         "mfma.hpp"),
                                fetch_kib=134327.7 + 268439.2 + 170149.6 + 994744.1,
                                write_kib=143909.4 + 786490.1 + 786461.9 + 542284.8,
                                sha256=_BWD_SHA),
    "qk_prologue_kernel": dict(sources=("layer_io.hip", "mfma.hpp"), fetch_kib=131099.8,
                               write_kib=262144.0, sha256=_LIO_SHA),
    "output_epilogue_kernel": dict(sources=("layer_io.hip", "mfma.hpp"), fetch_kib=131096.9,
                                   write_kib=131072.0, sha256=_LIO_SHA),
    "gates_kernel": dict(sources=("gates.hip",), fetch_kib=4114.0, write_kib=8192.0,
                         sha256="2bde382d2f924a1318325130cdb94dab"
                         "7d2b47dcae9f102ec3b939b9dde52ce6"),
}


# MFMA-pipe busy fraction from rocprofv3 counters (SQ_VALU_MFMA_BUSY_CYCLES summed over the
# 1,024 SIMDs / (GRBM_GUI_ACTIVE per XCD x 1,024), per dispatch, averaged), with the sources
# they were taken at (profiles/mfma_counters_B8H16T4096d128.md); null once the sources differ.
# It is the fraction of the kernel's duration the matrix pipes were busy, at the clock the GPU
# ran, beside the FLOP-derived fraction of the datasheet peak.
MFMA_BUSY = {
    "chunk_fwd_fused_kernel": dict(sources=TRAFFIC["chunk_fwd_fused_kernel"]["sources"],
                                   busy=0.415, sha256=TRAFFIC["chunk_fwd_fused_kernel"]["sha256"]),
    "chunk_scan_bf16_kernel": dict(sources=TRAFFIC["chunk_scan_bf16_kernel"]["sources"],
                                   busy=0.293, sha256=_SPLIT_SHA),
    "chunk_prep_kernel": dict(sources=TRAFFIC["chunk_prep_kernel"]["sources"], busy=0.111,
                              sha256=_SPLIT_SHA),
}


def mfma_busy(kernel):
    t = MFMA_BUSY.get(kernel) if kernel else None
    if t is None or sources_sha256(t["sources"]) != t["sha256"]:
        return None
    return t["busy"]


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes(kernel):
    """Counter-derived HBM bytes per launch, or None when the kernel changed since."""
    t = TRAFFIC.get(kernel) if kernel else None
    if t is None or t["sha256"] is None or sources_sha256(t["sources"]) != t["sha256"]:
        return None
    return round(t["fetch_kib"] * 1024 * FETCH_FACTOR + t["write_kib"] * 1024 * WRITE_FACTOR)


def roofline_of(kernel, us, flop, nbytes):
    """The roof that bounds a kernel is the one its algorithmic work reaches last."""
    t_mfma = flop / PEAK_BF16_FLOPS
    t_hbm = nbytes / PEAK_HBM_BPS
    sec = us * 1e-6
    if t_hbm >= t_mfma:
        r = {"bound": "hbm", "achieved": nbytes / sec / 1e9, "peak": PEAK_HBM_BPS / 1e9,
             "unit": "GB/s", "frac": nbytes / sec / PEAK_HBM_BPS}
    else:
        r = {"bound": "mfma", "achieved": flop / sec / 1e12, "peak": PEAK_BF16_FLOPS / 1e12,
             "unit": "TFLOP/s", "frac": flop / sec / PEAK_BF16_FLOPS}
    r["traffic"] = traffic_bytes(kernel)
    r.update({"kernel": kernel, "us": us, "algorithmic_bytes": nbytes, "algorithmic_flop": flop,
              "mfma_frac": flop / sec / PEAK_BF16_FLOPS, "hbm_frac": nbytes / sec / PEAK_HBM_BPS,
              "mfma_busy_counter": mfma_busy(kernel)})
    return r


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle", type=float, default=0.3,
                   help="seconds of untimed calls before each timed section")
    p.add_argument("--decode-steps", type=int, default=64)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-backward", action="store_true")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-peaks", action="store_true")
    p.add_argument("--no-configs", action="store_true")
    p.add_argument("--cpu-configs", action="store_true",
                   help="also time the oracle on every config (about a minute of CPU)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def up(x, dtype):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype)


def settle(torch, fns, seconds):
    """Untimed repetitions of the callables for about `seconds` of wall time,
    so that the GPU clock has left its idle state before anything is timed
    (a few steps from idle run up to 20% slower than the steady state)."""
    t0 = time.perf_counter()
    while True:
        for _ in range(10):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def time_calls(torch, fns, steps):
    """Mean time (ms) of each of the callables in `fns`, launched in order
    `steps` times on the current stream, from HIP events recorded between
    them; and the time per step of `steps` steps run back to back, bracketed
    by a synchronisation and one HIP event on each side (no events between
    the steps: each event is a marker the GPU processes between kernels,
    which added about 5 us per step when recorded around every call)."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        ev[s][0].record()
        for i, fn in enumerate(fns):
            fn()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    means = [sum(e[i].elapsed_time(e[i + 1]) for e in ev) / steps for i in range(len(fns))]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        for fn in fns:
            fn()
    e1.record()
    torch.cuda.synchronize()
    span = e0.elapsed_time(e1) / steps
    return means, span


def bench_forward(args, torch, si, mdn):
    import numpy as np
    cfg = si.CONFIGS[2]
    t0 = time.time()
    inp = si.make_forward(cfg)
    log(f"inputs {cfg.name} drawn in {time.time() - t0:.1f}s")
    bf = torch.bfloat16
    f32 = torch.float32
    plan = mdn.ChunkPlan(up(inp["q"], bf), up(inp["k"], bf), up(inp["v"], bf),
                         up(inp["alpha"], f32), up(inp["mu"], f32), up(inp["eta"], f32))
    toh = cfg.B * cfg.T * cfg.H
    heads = cfg.B * cfg.H
    tokens = cfg.B * cfg.T
    # the step: one mdn_chunk_fwd, which for bf16 launches chunk_coef_kernel
    # (about 6% of the call) and then chunk_fwd_fused_kernel; the events bracket the
    # call, so the fused kernel's rate below includes the coefficient kernel's
    # time (it is understated, never overstated)
    settle(torch, [plan.forward], args.settle)
    for _ in range(args.warmup):
        plan.forward()
    (fwd_ms,), step_ms = time_calls(torch, [plan.forward], args.steps)
    log(f"forward: {step_ms * 1e3:.1f} us/step (call {fwd_ms * 1e3:.1f} us)")
    flush_ab = bench_flush_ab(args, torch, plan)
    kernels = {
        "chunk_fwd_fused_kernel": roofline_of("chunk_fwd_fused_kernel", fwd_ms * 1e3,
                                              FLOP_FWD * toh,
                                              BYTES_FWD * toh + STATE_BYTES_HEAD * heads),
    }
    kernels["chunk_fwd_fused_kernel"]["timed_with"] = "chunk_coef_kernel (same call)"
    # the same forward through the exported two-phase entry points
    settle(torch, [plan.prepare, plan.scan], args.settle)
    (prep_ms, scan_ms), split_ms = time_calls(torch, [plan.prepare, plan.scan], args.steps)
    log(f"split path: prepare {prep_ms * 1e3:.1f} us, scan {scan_ms * 1e3:.1f} us")
    split = {
        "us_per_step": split_ms * 1e3, "tokens_per_s": tokens / (split_ms * 1e-3),
        "chunk_prep_kernel": roofline_of("chunk_prep_kernel", prep_ms * 1e3, FLOP_PREP * toh,
                                         BYTES_PREP * toh),
        "chunk_scan_bf16_kernel": roofline_of("chunk_scan_bf16_kernel", scan_ms * 1e3,
                                              FLOP_SCAN * toh,
                                              BYTES_SCAN * toh + STATE_BYTES_HEAD * heads),
    }
    roofline = dict(kernels["chunk_fwd_fused_kernel"])
    fwd = {"us_per_step": step_ms * 1e3, "tokens_per_s": tokens / (step_ms * 1e-3),
           "mfma_frac": FLOP_FWD * toh / (step_ms * 1e-3) / PEAK_BF16_FLOPS,
           "hbm_frac_algorithmic": (BYTES_FWD * toh + STATE_BYTES_HEAD * heads)
           / (step_ms * 1e-3) / PEAK_HBM_BPS, "_flush_ab": flush_ab}
    # the same layer in the four-gate form: an explicit update-step gate beta
    # (one more fp32 gate per token and head to read)
    beta = si.make_forward(cfg, beta="logit")["beta"]
    plan_b = mdn.ChunkPlan(*plan.args, beta=up(beta, f32))
    del beta
    settle(torch, [plan_b.forward], args.settle)
    for _ in range(args.warmup):
        plan_b.forward()
    _, beta_ms = time_calls(torch, [plan_b.forward], args.steps)
    log(f"forward with a beta gate: {beta_ms * 1e3:.1f} us/step")
    fwd["beta_gate"] = {"workload": "the same layer with beta = sigmoid(z), z ~ N(0, 1)",
                        "us_per_step": beta_ms * 1e3, "tokens_per_s": tokens / (beta_ms * 1e-3),
                        "hbm_frac_algorithmic": (BYTES_FWD_BETA * toh + STATE_BYTES_HEAD * heads)
                        / (beta_ms * 1e-3) / PEAK_HBM_BPS}
    del plan_b
    # the same layer saving every token's residual for a backward pass
    plan_s = mdn.ChunkPlan(*plan.args, save_vt=True)
    settle(torch, [plan_s.forward], args.settle)
    for _ in range(args.warmup):
        plan_s.forward()
    _, save_ms = time_calls(torch, [plan_s.forward], args.steps)
    log(f"forward saving the residuals: {save_ms * 1e3:.1f} us/step")
    fwd["save_residuals"] = {"workload": "the same layer also writing Vt [B, T, H, Dv] (bf16)",
                             "us_per_step": save_ms * 1e3,
                             "tokens_per_s": tokens / (save_ms * 1e-3)}
    del plan_s
    # the gated delta rule: no mu (mu = 0), the momentum-free kernel
    a_, e_ = plan.args[3], plan.args[5]
    plan_g = mdn.ChunkPlan(plan.args[0], plan.args[1], plan.args[2], a_, None, e_)
    settle(torch, [plan_g.forward], args.settle)
    for _ in range(args.warmup):
        plan_g.forward()
    _, gdn_ms = time_calls(torch, [plan_g.forward], args.steps)
    log(f"forward with no mu (gated delta rule): {gdn_ms * 1e3:.1f} us/step")
    fwd["no_mu"] = {"workload": "the same layer with mu = 0 (no mu given): the gated delta rule",
                    "us_per_step": gdn_ms * 1e3, "tokens_per_s": tokens / (gdn_ms * 1e-3)}
    del plan_g
    # the coupled gates from logits (one mdn_gates_from_logits call), then the
    # four-gate forward on its outputs: the whole layer core from projections
    z = si.gate_logits(toh, seed=3, scale=1.0)
    shape = (cfg.B, cfg.T, cfg.H)
    zt = [up(z[n], f32).reshape(shape) for n in ("z_eta", "z_alpha", "z_beta", "z_mu")]
    del z
    gp = dict(tau=GATE_TAU, s=1.0, a=1.0, b=0.0, log_mu_min=-2.0)
    gates = mdn.gates_from_logits(*zt, **gp)
    gfn = lambda: mdn.gates_from_logits(*zt, **gp, out=gates)
    plan_z = mdn.ChunkPlan(*plan.args[:3], gates[0], gates[1], gates[2], beta=gates[3])
    settle(torch, [gfn, plan_z.forward], args.settle)
    for _ in range(args.warmup):
        gfn()
        plan_z.forward()
    (g_ms, _), gz_ms = time_calls(torch, [gfn, plan_z.forward], args.steps)
    gbs = BYTES_GATES * toh / (g_ms * 1e-3) / 1e9
    log(f"gates from logits: {g_ms * 1e3:.1f} us ({gbs:.0f} GB/s); with the forward "
        f"{gz_ms * 1e3:.1f} us/step")
    kernels["gates_kernel"] = roofline_of("gates_kernel", g_ms * 1e3, 0, BYTES_GATES * toh)
    fwd["from_logits"] = {"workload": "mdn_gates_from_logits (tau = sqrt(2048 / 16), s = a = 1, "
                                      "b = 0, log mu floor -2, logits ~ N(0, 1)) then the "
                                      "four-gate forward",
                          "us_per_step": gz_ms * 1e3, "tokens_per_s": tokens / (gz_ms * 1e-3),
                          "gates_us": g_ms * 1e3, "gates_GB_per_s": gbs}
    del plan_z, gates, zt
    # the layer's elementwise steps around the core: the query correction and
    # q, k normalisation before it, the gated RMSNorm after it
    q_, k_ = plan.args[0], plan.args[1]
    qn, kn = torch.empty_like(q_), torch.empty_like(k_)
    dcorr = torch.full((cfg.H,), 0.5, dtype=f32, device="cuda")
    gt = up(si.round_io(np.random.default_rng(5).standard_normal(plan.O.shape), "bf16"), bf)
    wn = torch.ones(cfg.Dv, dtype=f32, device="cuda")
    yo = torch.empty_like(plan.O)
    pro = lambda: mdn.qk_prologue(q_, k_, dcorr, out=(qn, kn))
    epi = lambda: mdn.output_epilogue(plan.O, gt, wn, out=yo)
    plan_n = mdn.ChunkPlan(qn, kn, *plan.args[2:6])
    settle(torch, [pro, plan_n.forward, epi], args.settle)
    (p_ms, _, e_ms), layer_ms = time_calls(torch, [pro, plan_n.forward, epi], args.steps)
    p_gbs = BYTES_PROLOGUE * toh / (p_ms * 1e-3) / 1e9
    e_gbs = BYTES_EPILOGUE * toh / (e_ms * 1e-3) / 1e9
    log(f"prologue {p_ms * 1e3:.1f} us ({p_gbs:.0f} GB/s), epilogue {e_ms * 1e3:.1f} us "
        f"({e_gbs:.0f} GB/s); prologue + forward + epilogue {layer_ms * 1e3:.1f} us/step")
    kernels["qk_prologue_kernel"] = roofline_of("qk_prologue_kernel", p_ms * 1e3, 0,
                                                BYTES_PROLOGUE * toh)
    kernels["output_epilogue_kernel"] = roofline_of("output_epilogue_kernel", e_ms * 1e3, 0,
                                                    BYTES_EPILOGUE * toh)
    fwd["with_prologue_epilogue"] = {
        "workload": "mdn_qk_prologue (d = 0.5 per head), the forward on its outputs, "
                    "mdn_output_epilogue (gate ~ N(0, 1), unit weight)",
        "us_per_step": layer_ms * 1e3, "tokens_per_s": tokens / (layer_ms * 1e-3),
        "prologue_us": p_ms * 1e3, "prologue_GB_per_s": p_gbs,
        "epilogue_us": e_ms * 1e3, "epilogue_GB_per_s": e_gbs}
    del plan_n, qn, kn, gt, yo
    return cfg, inp, step_ms, kernels, roofline, fwd, split


def bench_backward(args, torch, si, mdn, cfg, inp):
    """mdn_chunk_bwd on the headline layer with dO ~ N(0, 1) and no terminal
    state gradients; every gradient (q, k, v, alpha, mu, eta) computed.  The
    main figure takes the residuals the forward saved (the pages' trade); the
    recompute figure passes none and re-solves for them."""
    bf, f32 = torch.bfloat16, torch.float32
    cot = si.backward_cotangents(cfg, 12, terminal=False)
    args_ = (up(inp["q"], bf), up(inp["k"], bf), up(inp["v"], bf), up(inp["alpha"], f32),
             up(inp["mu"], f32), up(inp["eta"], f32), None, None, up(cot["dO"], bf))
    del cot
    B, T, H = cfg.B, cfg.T, cfg.H
    ws = torch.empty(mdn.workspace_bytes_bwd(B, T, H, cfg.Dk, cfg.Dv, bf), dtype=torch.uint8,
                     device="cuda")
    Vt = torch.empty_like(args_[2])
    mdn.chunk_fwd(*args_[:8], Vt=Vt)
    steps = max(1, args.steps // 5)
    toh = B * T * H
    flop_saved = FLOP_BWD_SAVED * toh
    flop = FLOP_BWD * toh
    out = {}
    for name, kw in (("saved", dict(Vt=Vt)), ("recompute", {})):
        fn = lambda: mdn.chunk_bwd(*args_, workspace=ws, state_grads=False, **kw)
        settle(torch, [fn], args.settle)
        for _ in range(max(1, args.warmup // 2)):
            fn()
        (_,), span = time_calls(torch, [fn], steps)
        out[name] = span * 1e3
    us, us_re = out["saved"], out["recompute"]
    tf = flop_saved / (us * 1e-6) / 1e12
    fb = FLOP_BWD_BF16_SAVED * toh
    peak_saved, peak_re = mixed_peak(flop_saved, fb), mixed_peak(flop, FLOP_BWD_BF16 * toh)
    log(f"backward: {us:.1f} us/step with saved residuals ({tf:.1f} TFLOP/s of dense work, "
        f"mixed peak {peak_saved / 1e12:.1f}), {us_re:.1f} us/step recomputing them")
    return {"workload": f"mdn_chunk_bwd on {cfg.name}: dO ~ N(0, 1), all gradients, the "
                        "forward's saved residuals; both scans and most per-chunk products on bf16 "
                        "MFMA, the rest fp32 (fp32 MFMA)",
            "us_per_step": us, "tokens_per_s": B * T / (us * 1e-6), "steps_timed": steps,
            "recompute_us_per_step": us_re,
            "recompute_tokens_per_s": B * T / (us_re * 1e-6),
            "roofline": {"bound": "mfma", "achieved": tf, "peak": peak_saved / 1e12,
                         "unit": "TFLOP/s", "frac": flop_saved / (us * 1e-6) / peak_saved,
                         "peak_of": "mix: the bf16 products at the bf16 peak (2.5 PFLOP/s), "
                                    "the rest at the fp32 matrix peak (157.3 TFLOP/s)",
                         "algorithmic_flop_bf16": fb,
                         "traffic": traffic_bytes("chunk_bwd"), "algorithmic_flop": flop_saved,
                         "algorithmic_bytes": BYTES_BWD_SAVED * toh,
                         "hbm_frac": BYTES_BWD_SAVED * toh / (us * 1e-6) / PEAK_HBM_BPS},
            "recompute_roofline": {"bound": "mfma", "achieved": flop / (us_re * 1e-6) / 1e12,
                                   "peak": peak_re / 1e12, "unit": "TFLOP/s",
                                   "frac": flop / (us_re * 1e-6) / peak_re,
                                   "traffic": traffic_bytes("chunk_bwd_recompute"),
                                   "algorithmic_flop": flop,
                                   "algorithmic_bytes": BYTES_BWD * toh}}


def bench_decode(args, torch, si, mdn):
    cfg = si.CONFIGS[4]
    import dataclasses
    dcfg = dataclasses.replace(cfg, steps=args.decode_steps)
    t0 = time.time()
    stream = si.decode_stream(dcfg)
    S0, M0 = next(stream)
    S = up(S0, torch.float32)
    M = up(M0, torch.float32)
    del S0, M0
    bf, f32 = torch.bfloat16, torch.float32
    toks = []
    for _ in range(dcfg.steps):
        t = next(stream)
        toks.append((up(t["q"], bf), up(t["k"], bf), up(t["v"], bf), up(t["alpha"], f32),
                     up(t["mu"], f32), up(t["eta"], f32)))
    o = torch.empty((cfg.N, cfg.H, cfg.Dv), dtype=bf, device="cuda")
    log(f"decode inputs ({dcfg.steps} steps) drawn in {time.time() - t0:.1f}s")
    settle(torch, [lambda: mdn.decode_step(*toks[0], S, M, o)], args.settle)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in toks:
        mdn.decode_step(*t, S, M, o)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / dcfg.steps * 1e3
    heads = cfg.N * cfg.H
    gbs = DEC_BYTES_HEAD * heads / (us * 1e-6) / 1e9
    log(f"decode: {us:.1f} us/step, {gbs:.0f} GB/s algorithmic")
    # the gated delta rule: no mu and no momentum state, S alone streams
    settle(torch, [lambda: mdn.decode_step(*toks[0][:4], None, toks[0][5], S, None, o)],
           args.settle)
    e0.record()
    for t in toks:
        mdn.decode_step(*t[:4], None, t[5], S, None, o)
    e1.record()
    torch.cuda.synchronize()
    us_g = e0.elapsed_time(e1) / dcfg.steps * 1e3
    gbs_g = DEC_BYTES_HEAD_GDN * heads / (us_g * 1e-6) / 1e9
    log(f"decode with no mu and no M: {us_g:.1f} us/step, {gbs_g:.0f} GB/s algorithmic")
    return {"workload": f"decode N{cfg.N} H{cfg.H} d{cfg.Dk} fp32 state, bf16 tokens",
            "us_per_step": us, "GB_per_s": gbs, "hbm_frac": gbs * 1e9 / PEAK_HBM_BPS,
            "bytes_per_step": DEC_BYTES_HEAD * heads, "steps_timed": dcfg.steps,
            "kernel": "decode_step_kernel", "traffic": traffic_bytes("decode_step_kernel"),
            "no_mu": {"workload": "the same steps with mu = 0 and no momentum state",
                      "us_per_step": us_g, "GB_per_s": gbs_g,
                      "hbm_frac": gbs_g * 1e9 / PEAK_HBM_BPS,
                      "bytes_per_step": DEC_BYTES_HEAD_GDN * heads}}


# tokens/s against sequence length at a fixed 16,384 tokens per call (T x B), H = 16, d = 128,
# gates as in the headline layer; the last point is the 16K-context layer
SWEEP = [(2048, 8), (4096, 4), (8192, 2), (16384, 1)]


def bench_sweep(args, torch, si, mdn):
    import dataclasses
    base = si.CONFIGS[2]
    out = []
    for T, B in SWEEP:
        cfg = dataclasses.replace(base, name=f"sweep-bf16-B{B}H16T{T}d128", B=B, T=T,
                                  seed=si.SEED_BASE + 100 + T // 1024)
        inp = si.make_forward(cfg)
        bf, f32 = torch.bfloat16, torch.float32
        plan = mdn.ChunkPlan(up(inp["q"], bf), up(inp["k"], bf), up(inp["v"], bf),
                             up(inp["alpha"], f32), up(inp["mu"], f32), up(inp["eta"], f32))
        del inp
        settle(torch, [plan.forward], args.settle)
        for _ in range(args.warmup):
            plan.forward()
        (call_ms,), step_ms = time_calls(torch, [plan.forward], args.steps)
        wg = B * cfg.H * (cfg.Dv // 64)
        nseg = mdn.segment_count(B, T, cfg.H, cfg.Dk, cfg.Dv, True)
        path = (f"segments ({nseg})" if nseg else
                "row_split" if wg <= mdn.ROW_SPLIT_MAX_TILES else "column_tiles")
        out.append({"T": T, "B": B, "H": cfg.H, "us_per_step": step_ms * 1e3,
                    "tokens_per_s": B * T / (step_ms * 1e-3), "column_tiles": wg, "path": path})
        log(f"sweep T{T} B{B}: {step_ms * 1e3:.1f} us/step, {B * T / (step_ms * 1e-3):.3e} tokens/s, "
            f"{wg} column tiles, {path}")
        del plan
    return {"workload": "mdn_chunk_fwd, T x B = 16384 tokens per call, H16 d128, bf16",
            "bound": "the column tiles run one workgroup per (b, h, 64 value columns) through "
                     "its chunks in sequence, so fewer than 256 of them leave CUs idle; the "
                     "segment scan (the default for few heads and long sequences) walks about "
                     "2 / nseg of the chunks in sequence",
            "points": out}


def bench_peaks(args, torch):
    """Measured ceilings on this GPU: a dense bf16 MFMA loop (8 independent
    16x16x32 chains per wavefront, 4 wavefronts per workgroup) and a 2 GiB
    streaming copy (cached and non-temporal accesses)."""
    from chunkwise_delta_rule_amd import peaks
    out = torch.empty(4096 * 256, dtype=torch.float32, device="cuda")
    wg, iters = 4096, 2048
    fn = lambda: peaks.mfma_bf16(wg, iters, out)
    flop = fn()
    settle(torch, [fn], args.settle)
    (ms,), _ = time_calls(torch, [fn], 10)
    mfma = flop / (ms * 1e-3)
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    copy = {}
    for nt in (True, False):
        cf = lambda: peaks.copy(src, dst, nontemporal=nt)
        nbytes = cf()
        settle(torch, [cf], args.settle)
        (cms,), _ = time_calls(torch, [cf], 10)
        copy["nontemporal" if nt else "cached"] = nbytes / (cms * 1e-3)
    del src, dst
    best = max(copy.values())
    log(f"measured peaks: bf16 MFMA {mfma / 1e12:.0f} TFLOP/s ({mfma / PEAK_BF16_FLOPS:.1%} of "
        f"the datasheet), copy {copy['nontemporal'] / 1e9:.0f} GB/s non-temporal, "
        f"{copy['cached'] / 1e9:.0f} GB/s cached ({best / PEAK_HBM_BPS:.1%})")
    return {"mfma_bf16_TFLOP_per_s": mfma / 1e12,
            "mfma_bf16_frac_of_datasheet": mfma / PEAK_BF16_FLOPS,
            "mfma_workload": f"{wg} workgroups x 4 wavefronts x {iters} rounds of 8 independent "
                             "v_mfma_f32_16x16x32_bf16",
            "copy_GB_per_s": {k: v / 1e9 for k, v in copy.items()},
            "copy_frac_of_datasheet": best / PEAK_HBM_BPS,
            "copy_workload": "2 GiB read + 2 GiB written, 16 B per lane, grid-stride",
            "datasheet": {"mfma_bf16_TFLOP_per_s": PEAK_BF16_FLOPS / 1e12,
                          "hbm_GB_per_s": PEAK_HBM_BPS / 1e9}}


def time_calls_each(torch, fn, steps, flush=None):
    """Median and mean time (ms) of single calls, each bracketed by its own
    events; with `flush`, that callable runs between the calls (outside the
    events)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        if flush is not None:
            flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2], sum(t) / len(t)


def bench_flush_ab(args, torch, plan):
    """The headline call timed one call at a time, back to back and with a
    1 GiB write between calls (evicting the 256 MB last-level cache), median
    of 20 each: whether data left in the cache by the previous call helps."""
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    flush = lambda: buf.fill_(0)
    settle(torch, [plan.forward], args.settle)
    med, mean = time_calls_each(torch, plan.forward, 20)
    settle(torch, [flush, plan.forward], args.settle)
    fmed, fmean = time_calls_each(torch, plan.forward, 20, flush=flush)
    del buf
    log(f"one call at a time: median {med * 1e3:.1f} us back to back, {fmed * 1e3:.1f} us "
        f"after a 1 GiB write")
    return {"median_us_back_to_back": med * 1e3, "mean_us_back_to_back": mean * 1e3,
            "median_us_after_1GiB_write": fmed * 1e3, "mean_us_after_1GiB_write": fmean * 1e3,
            "calls": 20}


def bench_configs(args, torch, si, mdn):
    """The other forward configurations at their own sizes: the 400M-like
    layer (B4 H8 T2048) and the 16K-context layer (B1 H16 T16384) as drawn
    and with no mu (the gated delta rule on the same inputs).  Each is timed
    under the three partitions of the state (column tiles, row split, segment
    scan); `us_per_step` is the one the default rule picks (the segment scan
    where three or more segments of at least 16 chunks fit (8 with no mu), else the row
    split up to 32 tiles of 64 value columns, else the column tiles)."""
    bf, f32 = torch.bfloat16, torch.float32
    out = {}
    # the fp32 case (one path: prepare, then the fp32 scan)
    cfg = si.CONFIGS[0]
    inp = si.make_forward(cfg)
    plan = mdn.ChunkPlan(up(inp["q"], f32), up(inp["k"], f32), up(inp["v"], f32),
                         up(inp["alpha"], f32), up(inp["mu"], f32), up(inp["eta"], f32))
    del inp
    settle(torch, [plan.forward], args.settle)
    for _ in range(args.warmup):
        plan.forward()
    (call_ms,), step_ms = time_calls(torch, [plan.forward], args.steps)
    del plan
    out["config0"] = {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "H": cfg.H,
                      "us_per_step": step_ms * 1e3,
                      "tokens_per_s": cfg.B * cfg.T / (step_ms * 1e-3),
                      "kernels": "chunk_prep_kernel<float>, chunk_scan_kernel<float>"}
    log(f"config0: {step_ms * 1e3:.1f} us/step")
    for key, cfg, mu_null in (("config1", si.CONFIGS[1], False),
                              ("config3_runA", si.CONFIGS[3], False),
                              ("config3_runB_no_mu", si.CONFIGS[3], True)):
        inp = si.make_forward(cfg)
        args_dev = (up(inp["q"], bf), up(inp["k"], bf), up(inp["v"], bf), up(inp["alpha"], f32),
                    None if mu_null else up(inp["mu"], f32), up(inp["eta"], f32))
        del inp
        toh = cfg.B * cfg.T * cfg.H
        heads = cfg.B * cfg.H
        tiles = heads * (cfg.Dv // 64)
        nseg_auto = mdn.segment_count(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, not mu_null)
        auto = ("segments" if nseg_auto else
                "row_split" if tiles <= mdn.ROW_SPLIT_MAX_TILES else "column_tiles")
        per_path = {}
        for path in ("column_tiles", "row_split", "segments"):
            with mdn.fwd_path(path):
                nseg = mdn.segment_count(cfg.B, cfg.T, cfg.H, cfg.Dk, cfg.Dv, not mu_null)
                if path == "segments" and nseg == 0:
                    continue
                plan = mdn.ChunkPlan(*args_dev)
                settle(torch, [plan.forward], args.settle)
                for _ in range(args.warmup):
                    plan.forward()
                (call_ms,), step_ms = time_calls(torch, [plan.forward], args.steps)
                del plan
            r = roofline_of(None, call_ms * 1e3, FLOP_FWD * toh,
                            BYTES_FWD * toh + STATE_BYTES_HEAD * heads)
            if path == "column_tiles":
                r["kernel"] = "chunk_fwd_fused_kernel" + ("<no mu>" if mu_null else "")
                r["timed_with"] = "chunk_coef_kernel (same call)"
            elif path == "row_split":
                r["kernel"] = "chunk_scan_rs_kernel" + ("<no mu>" if mu_null else "")
                r["timed_with"] = "chunk_prep_kernel (same call)"
            else:
                r["kernel"] = "chunk_fwd_seg_kernel" + ("<no mu>" if mu_null else "")
                r["timed_with"] = ("chunk_coef_kernel, the two passes and seg_combine_kernel "
                                   f"(same call; {nseg} segments)")
            # counter traffic of the whole call, recorded for the default path
            tkey = {("config1", "column_tiles"): "config1_fused",
                    ("config3_runA", "segments"): "config3_segments",
                    ("config3_runB_no_mu", "segments"): "config3_segments_no_mu"}.get((key, path))
            r["traffic"] = traffic_bytes(tkey)
            per_path[path] = {"us_per_step": step_ms * 1e3,
                              "tokens_per_s": cfg.B * cfg.T / (step_ms * 1e-3), "roofline": r}
            log(f"{key} {path}: {step_ms * 1e3:.1f} us/step, "
                f"{cfg.B * cfg.T / (step_ms * 1e-3):.3e} tokens/s")
        out[key] = {"workload": f"{cfg.name}{' with mu = 0 (no mu given)' if mu_null else ''}",
                    "B": cfg.B, "T": cfg.T, "H": cfg.H, "column_tiles": tiles,
                    "default_path": auto, "us_per_step": per_path[auto]["us_per_step"],
                    "tokens_per_s": per_path[auto]["tokens_per_s"],
                    "roofline": per_path[auto]["roofline"], "paths": per_path}
        del args_dev
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, cfg):
    import oracle
    lib = oracle.load()
    cores = oracle.max_threads(lib)
    # whole passes over the workload until about 10 s of CPU time have run (at
    # most 40 passes), so that the rate is not one short run's
    passes, sec = 0, 0.0
    while passes < 40 and (passes == 0 or sec < 10.0):
        t0 = time.perf_counter()
        oracle.recurrence(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["mu"], inp["eta"],
                          lib=lib)
        sec += time.perf_counter() - t0
        passes += 1
    log(f"oracle: {passes} passes, {sec:.1f}s on {cores} threads")
    return {"value": passes * cfg.B * cfg.T / sec, "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"the whole {cfg.name} workload (B{cfg.B} H{cfg.H} T{cfg.T} d{cfg.Dk}), "
                      f"fp64 token recurrence, {passes} passes, {sec:.1f}s"}


def cpu_configs(si):
    """The oracle timed on each config (the CPU-baseline leg, --cpu-configs):
    one whole pass of configs 0-3, and decode steps of config 4 until about
    5 s have run."""
    import oracle
    lib = oracle.load()
    cores = oracle.max_threads(lib)
    out = {}
    for i in range(4):
        cfg = si.CONFIGS[i]
        inp = si.make_forward(cfg)
        t0 = time.perf_counter()
        oracle.recurrence(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["mu"], inp["eta"],
                          inp.get("beta"), inp["S0"], inp["M0"], lib=lib)
        sec = time.perf_counter() - t0
        out[f"config{i}"] = {"seconds": sec, "tokens_per_s": cfg.B * cfg.T / sec,
                             "threads": cores, "sample": "one whole pass"}
        log(f"oracle config{i}: {sec:.2f}s on {cores} threads")
    cfg = si.CONFIGS[4]
    stream = si.decode_stream(cfg)
    S, M = next(stream)
    S = S.astype("float64")
    M = M.astype("float64")
    steps, sec = 0, 0.0
    while steps < cfg.steps and (steps == 0 or sec < 5.0):
        t = next(stream)
        t0 = time.perf_counter()
        _, S, M = oracle.decode_step(t["q"], t["k"], t["v"], t["alpha"], t["mu"], t["eta"], S, M,
                                     lib=lib)
        sec += time.perf_counter() - t0
        steps += 1
    out["config4"] = {"seconds_per_step": sec / steps, "head_steps_per_s":
                      steps * cfg.N * cfg.H / sec, "threads": cores,
                      "sample": f"{steps} of the {cfg.steps} decode steps"}
    log(f"oracle config4: {sec / steps:.3f}s per step on {cores} threads")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the MDN core shards "
              "over batch x heads with no communication, so the per-GPU figure is the "
              "--gpus 1 figure.", file=sys.stderr)
        sys.exit(2)
    import torch

    import synthetic_inputs as si
    from chunkwise_delta_rule_amd import mdn
    if not os.path.exists(mdn.LIB_PATH):
        from chunkwise_delta_rule_amd import build as libbuild
        libbuild.build()
    mdn.load_library()
    cfg, inp, step_ms, kernels, roofline, fwd, split = bench_forward(args, torch, si, mdn)
    flush_ab = fwd.pop("_flush_ab")
    backward = None if args.no_backward else bench_backward(args, torch, si, mdn, cfg, inp)
    decode = None if args.no_decode else bench_decode(args, torch, si, mdn)
    sweep = None if args.no_sweep else bench_sweep(args, torch, si, mdn)
    configs = None if args.no_configs else bench_configs(args, torch, si, mdn)
    peaks = None if args.no_peaks else bench_peaks(args, torch)
    base = None if args.no_cpu_baseline else cpu_baseline(inp, cfg)
    if base is not None and args.cpu_configs:
        base["per_config"] = cpu_configs(si)
    tokens = cfg.B * cfg.T
    line = {
        "metric": METRIC,
        "value": tokens / (step_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mdn_chunk_fwd 1.3B-like layer", "B": cfg.B, "T": cfg.T,
                   "H": cfg.H, "d_k": cfg.Dk, "d_v": cfg.Dv, "chunk": cfg.chunk,
                   "io": "bf16 q/k/v/O, fp32 gates and state", "tokens_per_step": tokens},
        "roofline": roofline,
        "forward": fwd,
        "kernels": kernels,
        "split_path": split,
        "backward": backward,
        "decode": decode,
        "timing_ab": flush_ab,
        "other_configs": configs,
        "sweep": sweep,
        "measured_peaks": peaks,
        "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
