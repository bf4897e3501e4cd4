// layer_io.hip -- the elementwise work around the MDN core, fused, on gfx950.
//
// "MDN: Parallelizing Stepwise Momentum for Delta Linear Attention" (slides),
// frame "The memory sits inside a familiar language-model block" (the paper's
// Sec. 3.3 and Fig. 3); the reading notes on the same paper, Sec. 2.9, spell
// the two steps out:
//   prologue  the Comba query correction q <- q - d k (d one coefficient per
//             head), then q and k L2-normalised per token and head:
//             x <- x / sqrt(sum x^2 + eps)
//   epilogue  the gated output norm before the output projection:
//             y = sigmoid(g) o (o / sqrt(mean o^2 + eps)) o w
//             per token and head over d_v, with one weight vector w [d_v]
//             shared by the heads; g is the caller's gate projection W_g x.
// The projections themselves (and the short convolution) carry trained
// weights and stay with the caller.
//
// Both are one pass over HBM: each row (one token and head, d = 64 or 128
// elements) is read once and written once.  A row is split over TPR lanes of
// one wavefront, 16 bytes per lane; the sums of squares are reduced across
// those lanes with shuffles, in fp32.
#include <hip/hip_runtime.h>

#include "mfma.hpp"

namespace mdn {
namespace {

template <typename E>
struct Vec16 {
    static constexpr int N = 16 / sizeof(E);
    float f[N];
    __device__ __forceinline__ void load(const E* p)
    {
        const uint4 w = *reinterpret_cast<const uint4*>(p);
        if constexpr (sizeof(E) == 2) {
            const unsigned u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = __uint_as_float(u[e] << 16);
                f[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
            }
        } else {
            f[0] = __uint_as_float(w.x);
            f[1] = __uint_as_float(w.y);
            f[2] = __uint_as_float(w.z);
            f[3] = __uint_as_float(w.w);
        }
    }
    __device__ __forceinline__ void store(E* p) const
    {
        if constexpr (sizeof(E) == 2) {
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(f[e]);
            *reinterpret_cast<bf16x8*>(p) = v;
        } else {
            *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
        }
    }
};

// sum over the TPR lanes that share a row (aligned groups of TPR lanes)
template <int TPR>
__device__ __forceinline__ float row_sum(float x)
{
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) x += __shfl_xor(x, o);
    return x;
}

template <typename E, int D>
__global__ __launch_bounds__(256) void qk_prologue_kernel(const E* __restrict__ q,
                                                          const E* __restrict__ k,
                                                          const float* __restrict__ dcorr,
                                                          E* __restrict__ qo, E* __restrict__ ko,
                                                          size_t rows, int H, float eps)
{
    constexpr int VE = Vec16<E>::N;
    constexpr int TPR = D / VE;                 // lanes per row
    const size_t nthreads = (size_t)gridDim.x * blockDim.x;
    const size_t t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    // every lane of a row group runs the same iterations (rows * TPR is a
    // multiple of TPR and so is the stride), so the shuffles stay in step
    for (size_t t = t0; t < rows * TPR; t += nthreads) {
        const size_t row = t / TPR;              // token * H + head
        const int c = (int)(t % TPR) * VE;
        const float dh = dcorr ? dcorr[row % H] : 0.f;
        Vec16<E> vq, vk;
        vq.load(q + row * D + c);
        vk.load(k + row * D + c);
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            vq.f[e] -= dh * vk.f[e];
            sq += vq.f[e] * vq.f[e];
            sk += vk.f[e] * vk.f[e];
        }
        const float rq = 1.f / sqrtf(row_sum<TPR>(sq) + eps);
        const float rk = 1.f / sqrtf(row_sum<TPR>(sk) + eps);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            vq.f[e] *= rq;
            vk.f[e] *= rk;
        }
        vq.store(qo + row * D + c);
        vk.store(ko + row * D + c);
    }
}

template <typename E, int D>
__global__ __launch_bounds__(256) void output_epilogue_kernel(const E* __restrict__ o,
                                                              const E* __restrict__ g,
                                                              const float* __restrict__ w,
                                                              E* __restrict__ y, size_t rows,
                                                              float eps)
{
    constexpr int VE = Vec16<E>::N;
    constexpr int TPR = D / VE;
    const size_t nthreads = (size_t)gridDim.x * blockDim.x;
    const size_t t0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    // the stride is a multiple of TPR, so a lane keeps its columns c .. c + VE - 1
    // for the whole loop: its weights are loaded once
    const int c = (int)(t0 % TPR) * VE;
    float wv[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) wv[e] = w ? w[c + e] : 1.f;
    for (size_t t = t0; t < rows * TPR; t += nthreads) {
        const size_t row = t / TPR;
        Vec16<E> vo, vg;
        vo.load(o + row * D + c);
        vg.load(g + row * D + c);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) ss += vo.f[e] * vo.f[e];
        const float r = 1.f / sqrtf(row_sum<TPR>(ss) * (1.f / D) + eps);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            // sigmoid with the hardware exponential and reciprocal
            const float gate = __builtin_amdgcn_rcpf(1.f + __expf(-vg.f[e]));
            vo.f[e] = gate * (vo.f[e] * r) * wv[e];
        }
        vo.store(y + row * D + c);
    }
}

constexpr unsigned LIO_MAX_BLOCKS = 8192;

unsigned grid_for(size_t threads)
{
    const size_t want = (threads + 255) / 256;
    return (unsigned)(want < 1 ? 1 : want > LIO_MAX_BLOCKS ? LIO_MAX_BLOCKS : want);
}

}  // namespace

// Host entries used by the C ABI layer; arguments are validated there.
hipError_t launch_qk_prologue(const void* q, const void* k, const float* dcorr, void* qo,
                              void* ko, size_t rows, int H, int D, bool bf16, float eps,
                              hipStream_t stream)
{
#define MDN_PRO(E, DD)                                                                         \
    if (D == DD) {                                                                             \
        constexpr int TPR = DD / Vec16<E>::N;                                                  \
        hipLaunchKernelGGL((qk_prologue_kernel<E, DD>), dim3(grid_for(rows * TPR)), dim3(256), \
                           0, stream, static_cast<const E*>(q), static_cast<const E*>(k),      \
                           dcorr, static_cast<E*>(qo), static_cast<E*>(ko), rows, H, eps);     \
        return hipGetLastError();                                                              \
    }
    if (bf16) {
        MDN_PRO(__bf16, 64) MDN_PRO(__bf16, 128)
    } else {
        MDN_PRO(float, 64) MDN_PRO(float, 128)
    }
#undef MDN_PRO
    return hipErrorInvalidValue;
}

hipError_t launch_output_epilogue(const void* o, const void* g, const float* w, void* y,
                                  size_t rows, int D, bool bf16, float eps, hipStream_t stream)
{
#define MDN_EPI(E, DD)                                                                          \
    if (D == DD) {                                                                              \
        constexpr int TPR = DD / Vec16<E>::N;                                                   \
        hipLaunchKernelGGL((output_epilogue_kernel<E, DD>), dim3(grid_for(rows * TPR)),         \
                           dim3(256), 0, stream, static_cast<const E*>(o),                      \
                           static_cast<const E*>(g), w, static_cast<E*>(y), rows, eps);         \
        return hipGetLastError();                                                               \
    }
    if (bf16) {
        MDN_EPI(__bf16, 64) MDN_EPI(__bf16, 128)
    } else {
        MDN_EPI(float, 64) MDN_EPI(float, 128)
    }
#undef MDN_EPI
    return hipErrorInvalidValue;
}

}  // namespace mdn
