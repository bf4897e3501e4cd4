// peaks.hip -- on-device ceilings the benchmark reports beside the datasheet
// peaks: a dense bf16 MFMA loop and a streaming copy through HBM.  Neither is
// part of the MDN path; they give the achieved fractions a measured ceiling
// on the machine at hand (its sustained clock, its HBM controller).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libmdn_peaks.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int CHAINS = 8;  // independent accumulators per wavefront

// Every wavefront issues `iters` rounds of CHAINS independent
// v_mfma_f32_16x16x32_bf16 (16,384 flop each); operands come from the thread
// index so nothing folds, and each lane writes one sum so nothing is dead.
__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float* __restrict__ out)
{
    const int tid = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = static_cast<__bf16>(1.0f + 1e-3f * static_cast<float>((tid + j) & 7));
        b[j] = static_cast<__bf16>(1e-3f * static_cast<float>((tid * 3 + j) & 15));
    }
    f32x4 acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[static_cast<size_t>(blockIdx.x) * blockDim.x + tid] = s;
}

// 16 bytes per lane per iteration, grid-stride; non-temporal loads and
// stores when `nt` (the data streams through once).
template <bool NT>
__global__ void __launch_bounds__(256) copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, size_t n)
{
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += stride) {
        if (NT) {
            u32x4 v = __builtin_nontemporal_load(src + i);
            __builtin_nontemporal_store(v, dst + i);
        } else {
            dst[i] = src[i];
        }
    }
}

}  // namespace

extern "C" {

int64_t mdn_peak_mfma_bf16_flop(int workgroups, int iters)
{
    if (workgroups <= 0 || iters <= 0) return 0;
    return static_cast<int64_t>(workgroups) * 4 /* wavefronts */ * iters * CHAINS * 16 * 16 *
           32 * 2;
}

int mdn_peak_mfma_bf16(int workgroups, int iters, float* out, hipStream_t stream)
{
    if (out == nullptr) return 1;
    if (workgroups <= 0 || iters <= 0) return 2;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, stream, iters, out);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

int mdn_peak_copy(const void* src, void* dst, size_t bytes, int nontemporal,
                  hipStream_t stream)
{
    if (src == nullptr || dst == nullptr) return 1;
    if (bytes % 16 != 0) return 2;
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0) return 4;
    const size_t n = bytes / 16;
    if (n == 0) return 0;
    const size_t want = (n + 255) / 256;
    const unsigned grid = static_cast<unsigned>(want < 16384 ? want : 16384);
    if (nontemporal)
        hipLaunchKernelGGL(copy_kernel<true>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    else
        hipLaunchKernelGGL(copy_kernel<false>, dim3(grid), dim3(256), 0, stream,
                           static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
