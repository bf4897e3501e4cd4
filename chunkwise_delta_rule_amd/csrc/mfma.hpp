// mfma.hpp -- matrix-core fragment helpers for gfx950 (CDNA4), wave64.
//
// Every dense contraction in libmdn is built from 16x16 output tiles of one
// MFMA instruction family per element type:
//   bf16: v_mfma_f32_16x16x32_bf16  (8 bf16 of A and of B per lane, fp32 acc)
//   fp32: v_mfma_f32_16x16x4_f32    (1 fp32 of A and of B per lane, fp32 acc)
//
// Operand convention used throughout ("both operands k-contiguous"):
//   D[i][n] += sum_k A[i][k] * B[k][n]
//   lane l supplies A[i0 + l%16][k0 + KW*(l/16) + j] and
//                   B[k0 + KW*(l/16) + j][n0 + l%16]   for j < KW,
// so an A fragment is KW consecutive elements of one row of a row-major A,
// and a B fragment is KW consecutive elements of one row of B^T.  A and B
// use the same (lane, j) -> k assignment, so the product does not depend on
// how the hardware orders k inside one instruction.
// The accumulator holds D[i0 + 4*(l/16) + r][n0 + l%16] in element r (0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mdn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

template <typename E>
struct Mma;

template <>
struct Mma<__bf16> {
    static constexpr int KSTEP = 32;  // k covered by one instruction
    static constexpr int KW = 8;      // k elements per lane
    static constexpr int PAD = 8;     // LDS row padding (elements): 16 bytes
    typedef bf16x8 frag;
    __device__ __forceinline__ static f32x4 mma(const frag& a, const frag& b, const f32x4& c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // KW consecutive elements at p (16-byte aligned)
    __device__ __forceinline__ static frag load(const __bf16* p)
    {
        return *reinterpret_cast<const bf16x8*>(p);
    }
    // KW elements p[j * stride] scaled by s[j] (fp32 product, rounded once)
    __device__ __forceinline__ static frag load_strided_scaled(const __bf16* p, int stride,
                                                               const float* s, float sign)
    {
        frag f;
#pragma unroll
        for (int j = 0; j < KW; ++j)
            f[j] = static_cast<__bf16>(sign * s[j] * static_cast<float>(p[j * stride]));
        return f;
    }
};

template <>
struct Mma<float> {
    static constexpr int KSTEP = 4;
    static constexpr int KW = 1;
    static constexpr int PAD = 4;     // 16 bytes
    typedef float frag;
    __device__ __forceinline__ static f32x4 mma(const frag& a, const frag& b, const f32x4& c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static frag load(const float* p) { return *p; }
    __device__ __forceinline__ static frag load_strided_scaled(const float* p, int, const float* s,
                                                               float sign)
    {
        return sign * s[0] * p[0];
    }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// element conversions
template <typename E>
__device__ __forceinline__ E to_elem(float x);
template <>
__device__ __forceinline__ __bf16 to_elem<__bf16>(float x) { return static_cast<__bf16>(x); }
template <>
__device__ __forceinline__ float to_elem<float>(float x) { return x; }

template <typename E>
__device__ __forceinline__ float to_f32(E x) { return static_cast<float>(x); }

// Store 4 consecutive elements (one accumulator's r = 0..3) at p.
template <typename E>
__device__ __forceinline__ void store4(E* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, float a, float b, float c, float d)
{
    bf16x4 v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    v[2] = static_cast<__bf16>(c);
    v[3] = static_cast<__bf16>(d);
    *reinterpret_cast<bf16x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d)
{
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

}  // namespace mdn
