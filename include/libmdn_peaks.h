/*
 * libmdn_peaks -- measured ceilings for the benchmark (not part of the MDN
 * path).  The benchmark reports each kernel's achieved rate against the
 * MI355X datasheet peaks (dense bf16 MFMA 2.5 PFLOP/s, HBM 8 TB/s) and, beside
 * them, against these two kernels run on the same GPU:
 *
 *   mdn_peak_mfma_bf16  every wavefront issues rounds of 8 independent
 *                       v_mfma_f32_16x16x32_bf16; flop per launch from
 *                       mdn_peak_mfma_bf16_flop.
 *   mdn_peak_copy       a grid-stride 16-byte-per-lane copy of `bytes` (read
 *                       once, written once), with non-temporal accesses when
 *                       `nontemporal` is nonzero.
 *
 * Pointers are device pointers owned by the caller; calls only enqueue work
 * on `stream`.  Status: 0 ok, 1 NULL pointer, 2 bad size, 4 misaligned
 * (16 bytes), 7 launch error.
 */
#ifndef LIBMDN_PEAKS_H
#define LIBMDN_PEAKS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Flop of one mdn_peak_mfma_bf16 launch (0 for non-positive arguments). */
int64_t mdn_peak_mfma_bf16_flop(int workgroups, int iters);

/* `workgroups` workgroups of 256 threads; `out` receives one float per
 * thread (workgroups * 256 floats). */
int mdn_peak_mfma_bf16(int workgroups, int iters, float* out, hipStream_t stream);

/* dst[0 .. bytes) = src[0 .. bytes); bytes a multiple of 16, both pointers
 * 16-byte aligned, the ranges disjoint. */
int mdn_peak_copy(const void* src, void* dst, size_t bytes, int nontemporal,
                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMDN_PEAKS_H */
