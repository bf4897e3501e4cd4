// chunk_common.hpp -- constants and LDS tile helpers shared by the chunkwise
// forward kernels (the two-phase prepare/scan path and the fused path).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfma.hpp"

namespace mdn {

constexpr int CH = 64;    // chunk length
constexpr int NT = 256;   // threads per workgroup (4 wavefronts)
constexpr int NVEC = 8;   // coefficient vectors per chunk in the workspace

// coefficient vector rows (each CH floats)
constexpr int V_ABAR = 0;   // abar_i                      (rows >= n: 0)
constexpr int V_AB1 = 1;    // alpha_i b_{i-1}             (rows >= n: 0)
constexpr int V_B = 2;      // b_i                         (rows >= n: 0)
constexpr int V_WS = 3;     // eta_j gamma_{n,j}           (cols >= n: 0)
constexpr int V_WM = 4;     // eta_j prod_{u=j+1}^{n} mu_u (cols >= n: 0)
constexpr int V_SCAL = 5;   // [abar_n, b_n, mubar_n]      (n = rows in this chunk)

// Accumulator slot -> physical chunk row used by the two-phase bf16 scan:
// inside each block of 32 rows, slots 4g + j and 16 + 4g + j hold rows
// 8g + j and 8g + 4 + j, so that a k-step fed from accumulator tiles 2s and
// 2s + 1 covers the 8 contiguous rows 32s + 8g + (0..7).
__device__ __forceinline__ int phys_row(int slot)
{
    const int q = slot & 31;
    return (slot & ~31) + 8 * ((q & 15) >> 2) + 4 * (q >> 4) + (q & 3);
}

// One direct global-to-LDS load of 16 bytes per lane: lane l's bytes land at
// lds_base + 16 l (lds_base is wave-uniform).
__device__ __forceinline__ void direct_load16(const void* gsrc, void* lds_base)
{
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// LDS layout of a 64-row bf16 tile with ROWB bytes per row (128 or 256).
// Rows are unpadded; every 1 KB group of rows (one direct load of 64 lanes x
// 16 bytes) is followed by PAD bytes, and inside a row the 16-byte chunks are
// XOR-permuted by (row & 3).  A fragment read by 16 lanes of rows
// phys_row(16 x + l16) -- rows r0 + {0..3, 8..11} or r0 + {4..7, 12..15} --
// then touches 8 distinct 16-byte bank groups per 8 lanes, and the address of
// step s is a per-row base plus 64 s bytes (an instruction immediate).
template <int ROWB>
struct TileLayout {
    static constexpr int G = 1024 / ROWB;               // rows per 1 KB group
    static constexpr int PAD = ROWB == 256 ? 32 : 64;   // bytes after each group
    static constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
    static constexpr int BYTES = CH * ROWB + (CH / G) * PAD;
    __device__ __forceinline__ static int row_base(int row)
    {
        return row * ROWB + (row / G) * PAD;
    }
    // byte offset of 16-byte logical chunk qc of row
    __device__ __forceinline__ static int chunk(int row, int qc)
    {
        return row_base(row) + 16 * (qc ^ (row & 3));
    }
    // Direct loads of rows [0, 64) of a row-major global tile (row stride in
    // elements) for wavefront `wave` of 4: instruction u fills group
    // 4 u + wave.  Since a group holds a multiple of 4 rows, the swizzle of a
    // lane's row depends on the lane only, so each lane's source offset is
    // one constant plus a wave-uniform group offset.  Rows >= n (a partial
    // last chunk) read row n - 1 instead.
    __device__ __forceinline__ static unsigned lane_offset(unsigned row_stride, int lane)
    {
        const int r = lane / CPR;
        return (unsigned)r * row_stride + 8u * (unsigned)((lane % CPR) ^ (r & 3));
    }
    __device__ __forceinline__ static void load(char* lds, const __bf16* __restrict__ g,
                                                unsigned row_stride, unsigned lane_off, int n,
                                                int wave, int lane)
    {
        constexpr int GROUPS = CH / G;
        static_assert(GROUPS % 4 == 0 && G % 4 == 0, "groups must split over 4 wavefronts");
        if (n == CH) {
#pragma unroll
            for (int u = 0; u < GROUPS / 4; ++u) {
                const int grp = 4 * u + wave;
                direct_load16(g + (unsigned)(grp * G) * row_stride + lane_off,
                              lds + grp * (1024 + PAD));
            }
        } else {
#pragma unroll
            for (int u = 0; u < GROUPS / 4; ++u) {
                const int grp = 4 * u + wave;
                const int row = grp * G + lane / CPR;
                const unsigned srow = (unsigned)min(row, n - 1);
                direct_load16(g + srow * row_stride + 8 * ((lane % CPR) ^ (row & 3)),
                              lds + grp * (1024 + PAD));
            }
        }
    }
};

// Workgroup barrier that orders LDS only: every wavefront's LDS writes
// before it are visible to every wavefront after it.  Unlike __syncthreads()
// it does not wait for outstanding global loads and stores, so register
// prefetches and output stores stay in flight across it; data that reaches
// LDS by direct global-to-LDS loads needs its own vmcnt wait before it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Each lane supplies the
// address of 4 consecutive 16-bit elements; inside every group of 16 lanes,
// lane i receives element (i % 4) of the values read by lanes 4 j + i / 4,
// j = 0..3, in that order.  So if lane 4 j + m of a group reads row r_j,
// columns c + 4 m .. + 3 of a row-major bf16 tile, lane i gets the column
// c + i entries of rows r_0..r_3: a 4-element k-fragment of the transpose.
__device__ __forceinline__ bf16x4 lds_read_tr4(const char* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4*)(p));
}

// D += A B for one 16x16x16 bf16 step: lane l supplies A[l % 16][4 (l / 16) + j]
// and B[4 (l / 16) + j][l % 16], j < 4; D as for the 16x16x32 form.
__device__ __forceinline__ f32x4 mma16(const bf16x4& a, const bf16x4& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

}  // namespace mdn
