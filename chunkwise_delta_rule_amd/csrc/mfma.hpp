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
//
// Accumulator-fed B operands ("k-permuted steps").  When the B operand of a
// product is itself the result of earlier 16x16 products still held in
// accumulators (B[k][n] in tiles of 16 k-rows), the k index of each step is
// taken in the order the accumulators already hold it:
//   bf16 step s: lane group g = l/16 supplies k = 32s + 4g + j (j < 4) and
//                k = 32s + 16 + 4g + (j - 4) (j >= 4): accumulator tiles 2s
//                and 2s + 1, elements 0..3 of each;
//   fp32 step s: k = 16 (s / 4) + 4g + (s % 4): tile s / 4, element s % 4.
// The B fragment is then a register move (plus a bf16 rounding), and the A
// fragment is read with the same k order (two 8-byte reads for bf16).
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
    // --- k-permuted steps -------------------------------------------------
    static constexpr int PERM_K = 32;          // k per step
    // first k row of element j of lane group g in step s
    __device__ __forceinline__ static int perm_row(int s, int g, int j)
    {
        return 32 * s + (j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4));
    }
    // A fragment of step s from a k-contiguous row p
    __device__ __forceinline__ static frag load_perm(const __bf16* p, int s, int g)
    {
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + 32 * s + 4 * g);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 32 * s + 16 + 4 * g);
        return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    // same, with the 4-element groups of the row XOR-permuted by x (a
    // multiple of 4)
    __device__ __forceinline__ static frag load_perm_xor(const __bf16* p, int s, int g, int x)
    {
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p + ((32 * s + 4 * g) ^ x));
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + ((32 * s + 16 + 4 * g) ^ x));
        return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    // B fragment of step s from accumulator tiles acc[2s], acc[2s + 1]
    __device__ __forceinline__ static frag from_acc(const f32x4* acc, int s)
    {
        const f32x4 a = acc[2 * s], b = acc[2 * s + 1];
        return frag{static_cast<__bf16>(a[0]), static_cast<__bf16>(a[1]),
                    static_cast<__bf16>(a[2]), static_cast<__bf16>(a[3]),
                    static_cast<__bf16>(b[0]), static_cast<__bf16>(b[1]),
                    static_cast<__bf16>(b[2]), static_cast<__bf16>(b[3])};
    }
    // same, element j scaled by w8[j] (the 8 scale factors of this lane's
    // k rows, contiguous)
    __device__ __forceinline__ static frag from_acc_scaled8(const f32x4* acc, int s,
                                                            const float* w8, float sign)
    {
        const f32x4 a = acc[2 * s], b = acc[2 * s + 1];
        const f32x4 wa = *reinterpret_cast<const f32x4*>(w8);
        const f32x4 wb = *reinterpret_cast<const f32x4*>(w8 + 4);
        return frag{static_cast<__bf16>(sign * wa[0] * a[0]), static_cast<__bf16>(sign * wa[1] * a[1]),
                    static_cast<__bf16>(sign * wa[2] * a[2]), static_cast<__bf16>(sign * wa[3] * a[3]),
                    static_cast<__bf16>(sign * wb[0] * b[0]), static_cast<__bf16>(sign * wb[1] * b[1]),
                    static_cast<__bf16>(sign * wb[2] * b[2]), static_cast<__bf16>(sign * wb[3] * b[3])};
    }
    // same, each k row scaled by w[k] (w indexed by absolute k row)
    __device__ __forceinline__ static frag from_acc_scaled(const f32x4* acc, int s, int g,
                                                           const float* w, float sign)
    {
        const f32x4 a = acc[2 * s], b = acc[2 * s + 1];
        const f32x4 wa = *reinterpret_cast<const f32x4*>(w + 32 * s + 4 * g);
        const f32x4 wb = *reinterpret_cast<const f32x4*>(w + 32 * s + 16 + 4 * g);
        return frag{static_cast<__bf16>(sign * wa[0] * a[0]), static_cast<__bf16>(sign * wa[1] * a[1]),
                    static_cast<__bf16>(sign * wa[2] * a[2]), static_cast<__bf16>(sign * wa[3] * a[3]),
                    static_cast<__bf16>(sign * wb[0] * b[0]), static_cast<__bf16>(sign * wb[1] * b[1]),
                    static_cast<__bf16>(sign * wb[2] * b[2]), static_cast<__bf16>(sign * wb[3] * b[3])};
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
    // --- k-permuted steps -------------------------------------------------
    static constexpr int PERM_K = 4;
    __device__ __forceinline__ static int perm_row(int s, int g, int)
    {
        return 16 * (s >> 2) + 4 * g + (s & 3);
    }
    __device__ __forceinline__ static frag load_perm(const float* p, int s, int g)
    {
        return p[perm_row(s, g, 0)];
    }
    __device__ __forceinline__ static frag from_acc(const f32x4* acc, int s)
    {
        return acc[s >> 2][s & 3];
    }
    __device__ __forceinline__ static frag from_acc_scaled(const f32x4* acc, int s, int g,
                                                           const float* w, float sign)
    {
        return sign * w[perm_row(s, g, 0)] * acc[s >> 2][s & 3];
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
