// chunk_fused.hip -- the chunkwise MDN forward for bf16 inputs on gfx950 as
// two launches: a small coefficient kernel (per chunk, fully parallel) and
// one fused kernel in which each chunk's Gram products, masks and triangular
// solve are formed in the same workgroup that carries the state, so T, A
// and the Gram matrices never leave LDS and q, k, v are read from HBM once.
//
// The method is the same as in chunk_fwd.hip ("MDN: Parallelizing Stepwise
// Momentum for Delta Linear Attention", slides Eqs. (7)-(9), (15)-(18),
// (40)-(42) in their Appendix C forms with the one-row-shifted residual mask;
// the reading notes on the same paper, Secs. 2.3-2.5).  Per chunk of C = 64
// rows with entry state (S0, M0), P = Diag(alpha) K, Khat = Diag(eta) K:
//   L  = I + (P Khat^T) o Gamma^-,   A = (Q Khat^T) o Gamma
//   R  = V - Diag(abar) K S0 + Diag(alpha_i b_{i-1}) K M0,   Vt = L^{-1} R
//   O  = Diag(abar) Q S0 - Diag(b) Q M0 + A Vt
//   S' = abar_C S0 - b_C M0 + K^T Diag(eta gamma_C) Vt
//   M' = mubar_C M0 - K^T Diag(eta mubar_C / mubar) Vt
//
// Two ways of evaluating the same quantities differ from chunk_fwd.hip:
//
//  * Gamma by 16-row blocks.  For a column j left of block I (rows
//    16 I .. 16 I + 15) the column recursion m_{i,j} = mu_i m_{i-1,j},
//    gamma_{i,j} = alpha_i gamma_{i-1,j} + m_{i,j} is affine in its value at
//    row 16 I - 1, so with the block-local products
//        ra_i = prod_{u=16I}^{i} alpha_u,   rp_i = prod_{u=16I}^{i} mu_u,
//        rg_i = alpha_i rg_{i-1} + rp_i     (rg_{16I-1} = 0)
//    it is gamma_{i,j} = ra_i gb_{I,j} + rg_i mb_{I,j} and m_{i,j} =
//    rp_i mb_{I,j}, where (gb, mb) are gamma and m at row 16 I - 1.  Only the
//    16 x 16 diagonal blocks run the recursion itself; every quantity stays a
//    sum of nonnegative products, with no division, so mu = 0 is exact.
//  * Vt = L^{-1} R by block forward substitution over the four 16-row blocks:
//        Vt_I = D_I (R_I - sum_{J<I} N_{IJ} Vt_J),  D_I = (I + N_{II})^{-1},
//    with N = L - I strictly lower triangular, so N_{II}^16 = 0 and
//    D_I = (I - N)(I + N^2)(I + N^4)(I + N^8): four levels of 16x16x16
//    products, all operands in registers.
//
// chunk_coef_kernel (one wavefront per chunk, lane = row and column index)
//   writes each chunk's tables: its gates, ra and rg of the rows, the
//   diagonal blocks of Gamma, (gb, mb) for every block and column, and the
//   six coefficient rows the scan reads.  Both value-column tiles of a head
//   use the same tables, which is why they are computed once, here.
//
// chunk_fwd_fused_kernel: 8 wavefronts for one (batch, head, 64 value columns).
//   compute 0..3  wavefront w keeps columns 16 w .. 16 w + 15 of S and M in
//                 fp32 accumulators for the whole sequence (rows of S in the
//                 permuted order phys_row(), as in chunk_fwd.hip) and works
//                 through chunk c: X = K [S|M], R, Q [S|M], the substitution,
//                 O^T (stored as 16-byte row pieces), the state update.
//   helper 4..7   helper h builds row block h of T and row block 3 - h of A.
//                 While chunk c is scanned it prepares chunk c + 1 in the
//                 other operand buffer (its V tile and coefficient rows by
//                 direct loads, its Gram products from the K and Q tiles in
//                 LDS, masked into -N, the block inverse D_h and A) and
//                 issues the direct loads of chunk c + 2's K and Q rows and
//                 tables.
// Synchronisation: one workgroup barrier per chunk, B0, once chunk c + 1 is
// complete and chunk c + 2's loads have landed, after which the compute
// wavefronts move on to chunk c + 1 and its buffer stops being written; one
// more at the start, for chunk 0's K, Q tiles and tables.
#include <hip/hip_runtime.h>

#include "chunk_common.hpp"
#include "mfma.hpp"

namespace mdn {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

template <int N>
struct IConst {
    static constexpr int value = N;
};

// Per-chunk coefficient tables (float offsets), as chunk_coef_kernel writes
// them to the workspace and the fused kernel keeps them in LDS (all but the
// coefficient rows, which go to the chunk's operand buffer).
struct ChunkTables {
    static constexpr int ALPHA = 0;           // gates of the rows
    static constexpr int RA = 64;             // block-local products of the rows
    static constexpr int RG = 128;
    // the three below are scaled by eta_j of their column j
    static constexpr int GB = 192;            // [3][64]: gamma at row 16 I - 1, column j (j < 16 I), I = 1..3
    static constexpr int MB = 384;            // [3][64]: m at row 16 I - 1
    static constexpr int GD = 576;            // Gamma's diagonal blocks, rows packed (gd_row)
    static constexpr int GD_ZERO = GD + 4 * 160;   // four zeros
    static constexpr int VEC = 1280;          // the six coefficient rows
    static constexpr int LDS_FLOATS = VEC;    // what the fused kernel keeps in LDS (5 KB)
    static constexpr int FLOATS = VEC + 6 * CH;
};

// Offset from ChunkTables::GD of row i (0..63) of Gamma's diagonal blocks.
// Block-local row r keeps columns 0 .. 4 ((r >> 2) + 1) - 1 of its block: the
// lower triangle, rounded up to whole 16-byte pieces (the entries above the
// diagonal in them are zero), 160 floats per block.
__host__ __device__ constexpr int gd_row(int i)
{
    const int r = i & 15, q = r >> 2;
    return 160 * (i >> 4) + 4 * (2 * q * (q + 1) + (r & 3) * (q + 1));
}
__host__ __device__ constexpr int gd_len(int i) { return 4 * (((i & 15) >> 2) + 1); }
static_assert(gd_row(15) + gd_len(15) == 160 && gd_row(63) + gd_len(63) == 640, "packed rows");
static_assert(ChunkTables::GD_ZERO + 4 <= ChunkTables::VEC, "tables overlap");

size_t chunk_fused_workspace_bytes(size_t nchunks)
{
    return nchunks * ChunkTables::FLOATS * sizeof(float);
}

// two 4-element k-fragments as one 8-element fragment (k of the second after
// the first's)
__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b)
{
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ bf16x4 lo4(const bf16x8& v) { return bf16x4{v[0], v[1], v[2], v[3]}; }
__device__ __forceinline__ bf16x4 hi4(const bf16x8& v) { return bf16x4{v[4], v[5], v[6], v[7]}; }

// LDS placement of the 16x16 blocks (x, J), J <= x, of T (-N below the block
// diagonal, D on it) and of A.  A block is stored in the lane order of the
// MFMA operand that reads it -- lane (l16, g) holds row 16 x + l16, columns
// 16 J + 4 g .. + 3, 8 bytes -- which is also the lane order of the helper
// accumulator that produces it, so every access is linear and free of bank
// conflicts.  Blocks read together share a 16-byte lane slot of a 1 KB pair
// area: (1,0|1,1), (2,0|2,1), (3,0|3,1), (3,2|3,3); the lone blocks (0,0) and
// (2,2) have 8-byte slots, 640 bytes apart, so that a read of both merged
// into one instruction reaches different banks.
struct FragSlot {
    int off;      // byte offset of lane 0's 8 bytes
    int stride;   // bytes from lane to lane
};
__host__ __device__ constexpr FragSlot frag_slot(int x, int J)
{
    return x == 0                ? FragSlot{4096, 8}
           : (x == 2 && J == 2) ? FragSlot{4096 + 640, 8}
                                : FragSlot{1024 * (x == 1 ? 0 : x == 2 ? 1 : J < 2 ? 2 : 3) + 8 * (J & 1), 16};
}
// bytes of one T or A area; 128 more than a multiple of 512, so that T and
// A blocks at equal offsets are never merged into one two-address access
constexpr int FRAG_AREA = 4096 + 640 + 512;

// x rounded to bf16 (nearest even).  Built from two packed 32-bit words: a
// 4-element bf16 vector built element by element and fed to a 16x16x16 MFMA
// is converted one element at a time (four conversions and two byte
// permutes instead of two packed conversions).
__device__ __forceinline__ unsigned pack_bf16(float a, float b)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_bit_cast(unsigned, bf16x2{static_cast<__bf16>(a), static_cast<__bf16>(b)});
}
__device__ __forceinline__ bf16x4 to_bf4(const f32x4& x)
{
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
    return __builtin_bit_cast(bf16x4, u32x2_t{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])});
}

// value of x in lane l (l uniform)
__device__ __forceinline__ float readlane_f(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// x of lane i - d within each row of 16 lanes; lanes i < d of a row get
// `fill` (DPP row_shr:d)
__device__ __forceinline__ float dpp_shr(float x, int d, float fill)
{
    int r = __float_as_int(fill);
    switch (d) {
    case 1: r = __builtin_amdgcn_update_dpp(r, __float_as_int(x), 0x111, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(r, __float_as_int(x), 0x112, 0xf, 0xf, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(r, __float_as_int(x), 0x114, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_update_dpp(r, __float_as_int(x), 0x118, 0xf, 0xf, false); break;
    }
    return __int_as_float(r);
}

// x in a VGPR, as a value the compiler must treat as new at this point.  An
// LDS address made this way stays the base of the accesses after it (their
// constant offsets become instruction immediates), instead of being
// re-derived, or rebased on a later access, from its parts.
__device__ __forceinline__ int opaque(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// ---------------------------------------------------------------------------
// Coefficient tables of every chunk.  A workgroup takes one chunk of up to
// 16 heads (workgroup g: chunk g % NC of batch row (g / NC) / NHG, heads
// 16 ((g / NC) % NHG) ..): it reads the gates of those heads and rows as
// contiguous memory (a head's own gates are H floats apart), stages them in
// LDS by head, and wavefront w then builds the tables of head w; lane l is
// row l (for the row quantities) and column l (for the column recursion);
// its 16-row block is l / 16.
constexpr int COEF_HEADS = 16;   // heads per workgroup, one wavefront each
constexpr int COEF_PITCH = CH + 4;   // LDS floats per head row (16-byte aligned, spreads banks)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(COEF_HEADS * 64) void chunk_coef_kernel(
    const float* __restrict__ alpha, const float* __restrict__ mu, const float* __restrict__ eta,
    const float* __restrict__ beta, float* __restrict__ ws, int T, int H, int NC, unsigned NHG)
{
    using CTb = ChunkTables;
    __shared__ __align__(16) float gates[4][COEF_HEADS][COEF_PITCH];   // alpha, mu, eta, beta
    // 32-bit indices: B NC NHG is below 2^32 (the entry points check it)
    const unsigned g = blockIdx.x / (unsigned)NC;
    const int c = (int)(blockIdx.x - g * (unsigned)NC);
    const int b = (int)(g / NHG), h0 = (int)(g - (unsigned)b * NHG) * COEF_HEADS;
    const int hg = min(COEF_HEADS, H - h0);            // heads of this workgroup
    const int n = min(CH, T - c * CH), last = n - 1;
    {
        // element e = row (e / hg) of head h0 + e % hg: consecutive threads read
        // consecutive floats; rows past a partial chunk's end repeat its last
        const size_t g0 = ((size_t)b * T + (size_t)c * CH) * H + h0;
        for (int e = threadIdx.x; e < CH * hg; e += COEF_HEADS * 64) {
            const int t = e / hg, hh = e - t * hg;
            const size_t gi = g0 + (size_t)min(t, last) * H + hh;
            gates[0][hh][t] = alpha[gi];
            gates[1][hh][t] = mu ? mu[gi] : 0.f;
            gates[2][hh][t] = eta[gi];
            gates[3][hh][t] = beta ? beta[gi] : 1.f;
        }
    }
    __syncthreads();
    // the wavefront index as a uniform value, so that the chunk's indices
    // and addresses are scalar arithmetic
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (wv >= hg) return;   // whole wavefronts; no barrier follows
    const int h = h0 + wv;
    const float ga = gates[0][wv][lane], gm = gates[1][wv][lane], ge = gates[2][wv][lane];
    const float gs = gates[3][wv][lane];
    float* tb = ws + (((size_t)b * H + h) * NC + c) * CTb::FLOATS;

    // Each table is stored as soon as it is known: every wavefront of the
    // grid is resident at once and runs the same steps in step, so stores
    // left to the end would leave the whole table write to one burst after
    // all the arithmetic instead of overlapping it.
    tb[CTb::ALPHA + lane] = ga;
    const int blk = lane >> 4, off = lane & 15;
    float ab[16], mbk[16], sbk[16];
#pragma unroll
    for (int t = 0; t < 16; t += 4) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&gates[0][wv][16 * blk + t]);
        const f32x4 m4 = *reinterpret_cast<const f32x4*>(&gates[1][wv][16 * blk + t]);
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(&gates[3][wv][16 * blk + t]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ab[t + e] = a4[e];
            mbk[t + e] = m4[e];
            sbk[t + e] = s4[e];
        }
    }
    // Block-local products of row `lane` (from its block's first row, row
    // included): ra = prod alpha, rp = prod mu,
    // rg_t = alpha_t rg_{t-1} + beta_t rp_t.  A range's triple composes
    // associatively -- earlier range L, later R:
    // (ra, rp, rg) = (ra_L ra_R, rp_L rp_R, ra_R rg_L + rp_L rg_R), a single
    // row being (alpha, mu, beta mu) -- so the prefixes are a 4-step scan
    // across the 16 lanes of the block.
    float ra = ga, rp = gm, rg = gs * gm;
#pragma unroll
    for (int d = 1; d < 16; d *= 2) {
        const float pa = dpp_shr(ra, d, 1.f), pp = dpp_shr(rp, d, 1.f), pg = dpp_shr(rg, d, 0.f);
        rg = ra * pg + pp * rg;
        ra = pa * ra;
        rp = pp * rp;
    }
    tb[CTb::RA + lane] = ra;
    tb[CTb::RG + lane] = rg;
    // the diagonal-block column recursion of column `lane` over its block's
    // rows: gamma_jj = beta_j, m_jj = 1; below the diagonal m_t = mu_t m_{t-1},
    // gamma_t = alpha_t gamma_{t-1} + beta_t m_t.  Every lane runs all 16 rows
    // from m = gamma = 0 and gets a 1 added to m on its diagonal row, which
    // starts the recursion there and leaves the rows above it at zero.
    // Stored (times the column's eta, as every use of the Gamma tables
    // wants) for the stored part of each row.
    float gam = 0.f, mm = 0.f;
    float gd[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        mm = mbk[t] * mm + (t == off ? 1.f : 0.f);
        gam = ab[t] * gam + sbk[t] * mm;
        gd[t] = gam;
        if (off < gd_len(t)) tb[CTb::GD + gd_row(16 * blk + t) + off] = ge * gam;
    }
    if (lane < 4) tb[CTb::GD_ZERO + lane] = 0.f;
    // block summaries (values at each block's last row)
    const float sa0 = readlane_f(ra, 15), sa1 = readlane_f(ra, 31), sa2 = readlane_f(ra, 47);
    const float sp0 = readlane_f(rp, 15), sp1 = readlane_f(rp, 31), sp2 = readlane_f(rp, 47);
    const float sg0 = readlane_f(rg, 15), sg1 = readlane_f(rg, 31), sg2 = readlane_f(rg, 47);
    // gamma, m of column `lane` at rows 16 I - 1 for the blocks below its own
    float gb = gam, mb = mm;
    float gbI[4] = {0.f, 0.f, 0.f, 0.f}, mbI[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int I = 1; I < 4; ++I) {
        if (I > 1) {   // through block I - 1 when the column lies left of it
            const float ca = I == 2 ? sa1 : sa2, cg = I == 2 ? sg1 : sg2, cp = I == 2 ? sp1 : sp2;
            const bool through = I > blk + 1;
            const float gn = ca * gb + cg * mb, mn = cp * mb;
            gb = through ? gn : gb;
            mb = through ? mn : mb;
        }
        gbI[I] = I > blk ? gb : 0.f;
        mbI[I] = I > blk ? mb : 0.f;
        tb[CTb::GB + 64 * (I - 1) + lane] = ge * gbI[I];
        tb[CTb::MB + 64 * (I - 1) + lane] = ge * mbI[I];
    }
    // chunk-level prefixes of row `lane`: the whole blocks before its own,
    // composed, then its block-local prefix; abar = prod alpha, mubar =
    // prod mu and b = the rg of the whole chunk (b_i = alpha_i b_{i-1} +
    // mubar_i is exactly rg's recursion from the chunk's first row)
    const float A1 = sa0, P1 = sp0, G1 = sg0;
    const float A2 = A1 * sa1, P2 = P1 * sp1, G2 = sa1 * G1 + P1 * sg1;
    const float A3 = A2 * sa2, P3 = P2 * sp2, G3 = sa2 * G2 + P2 * sg2;
    const float Ap = blk == 0 ? 1.f : blk == 1 ? A1 : blk == 2 ? A2 : A3;
    const float Pp = blk == 0 ? 1.f : blk == 1 ? P1 : blk == 2 ? P2 : P3;
    const float Gp = blk == 0 ? 0.f : blk == 1 ? G1 : blk == 2 ? G2 : G3;
    const float abar = Ap * ra;
    const float mubar = Pp * rp;
    const float bi = ra * Gp + Pp * rg;
    const float bprev = __shfl_up(bi, 1);
    const bool valid = lane < n;
    // gamma and m of column `lane` at the last row
    const int lb = last >> 4, tl = last & 15;
    float g_last = gd[15], m_last = mm;   // a full chunk: row 15 of block 3
    if (n < CH) {                         // the last chunk only
        float m2 = 1.f;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            m2 = t > off && t <= tl ? m2 * mbk[t] : m2;
            g_last = t == tl ? gd[t] : g_last;
        }
        m_last = tl >= off ? m2 : 0.f;
    }
    const float raL = readlane_f(ra, last), rgL = readlane_f(rg, last), rpL = readlane_f(rp, last);
    const float gbl = lb == 1 ? gbI[1] : lb == 2 ? gbI[2] : gbI[3];
    const float mbl = lb == 1 ? mbI[1] : lb == 2 ? mbI[2] : mbI[3];
    const float gl = blk < lb ? raL * gbl + rgL * mbl : blk == lb ? g_last : 0.f;
    const float ml = blk < lb ? rpL * mbl : blk == lb ? m_last : 0.f;
    const float abar_n = readlane_f(abar, last);
    const float b_n = readlane_f(bi, last);
    const float mbar_n = readlane_f(mubar, last);

    float* vec = tb + CTb::VEC;
    vec[V_ABAR * CH + lane] = valid ? abar : 0.f;
    vec[V_AB1 * CH + lane] = valid && lane > 0 ? ga * bprev : 0.f;
    vec[V_B * CH + lane] = valid ? bi : 0.f;
    vec[V_WS * CH + lane] = ge * gl;
    vec[V_WM * CH + lane] = ge * ml;
    vec[V_SCAL * CH + lane] = lane == 0 ? abar_n : lane == 1 ? b_n : lane == 2 ? mbar_n : 0.f;
}

// LDS layout of the K and Q tiles of the fused kernel (64 rows x DK bf16),
// filled by the helpers' direct loads.  Three accesses use it: 16-byte
// fragments of 16 consecutive rows at one 16-byte chunk (both waves' Gram
// and state products), transposing reads in which each 16-lane group takes
// four 8-byte pieces from each of 4 consecutive rows within one 64-byte
// window, and 16-byte lane stores (measured when the helpers still stored
// the rows from registers; the direct loads write it in 1 KB runs).  Rows
// are 2 DK + 32 bytes apart and the 16-byte chunks of a row are
// XOR-permuted by bits 2..3 of the row.
// Measured on gfx950 with every wavefront of a workgroup issuing each
// access, all three then run at the rate of a linear access of the same
// width; plain row strides of 2 DK or 2 DK + 64 bytes do not (the 16-row
// reads or the transposing reads take 1.6x to 3.7x as long).  The
// permutation touches chunk-index bits 0..1 only: step s of a fragment read
// is a fixed 64 s bytes further, and 16 rows further is a fixed J16 bytes.
template <int DK>
struct KQLayout {
    static constexpr int ROWB = 2 * DK;
    static constexpr int STRIDE = ROWB + 32;            // bytes from row to row
    static constexpr int BYTES = CH * STRIDE;
    static constexpr int J16 = 16 * STRIDE;
    static_assert(DK == 64 || DK == 128, "head size");
    __device__ __forceinline__ static int chunk(int row, int qc)
    {
        return row * STRIDE + 16 * (qc ^ ((row >> 2) & 3));
    }
};

// LDS of the fused kernel.  The V tile, T, A and the coefficient rows of a
// chunk live in operand buffer c & 1; K and Q in K/Q buffer c % 3: the
// helpers' direct loads of chunk c + 1's rows land while the compute
// wavefronts read chunk c - 1's and the helpers build chunk c's Gram
// products from chunk c's.  The tables of a chunk in table set c & 1.
template <int DK>
struct FusedLayout {
    using LK = KQLayout<DK>;                // K, Q: 64 rows x DK
    using LC = TileLayout<CH * 2>;          // V tile: 64 rows x 64
    static constexpr int OFF_V = 0;
    static constexpr int OFF_T = OFF_V + LC::BYTES;
    static constexpr int OFF_A = OFF_T + FRAG_AREA;
    static constexpr int OFF_VEC = OFF_A + FRAG_AREA;
    static constexpr int BUF = OFF_VEC + 6 * CH * 4;
    static constexpr int OFF_K = 2 * BUF;                 // three K buffers
    static constexpr int OFF_Q = OFF_K + 3 * LK::BYTES;   // three Q buffers
    static constexpr int TB_BYTES = ChunkTables::LDS_FLOATS * 4;
    static constexpr int OFF_TB = OFF_Q + 3 * LK::BYTES;  // two table sets
    static constexpr int BYTES = OFF_TB + 2 * TB_BYTES;
    static_assert(BYTES <= 160 * 1024, "LDS of one workgroup");
};

// The segment scan (layers with few heads).  The sequence is cut into nseg
// segments: segment 0 of ncs0 chunks, the others of ncs (the last may be
// shorter; see seg_lengths for why segment 0 is shorter).  The state map of a
// segment is affine: its exit pair (S, M) is its exit pair from a zero entry
// (the local part) plus a linear map Phi_s of its entry pair, and Phi_s is
// found by running the chunk recurrence with V = 0 from the columns of the
// identity.  Pass A runs segment 0 from the given entry state (with outputs)
// beside the local parts and maps of segments 1 .. nseg - 2; a small kernel
// then composes the entry states of segments 2 .. nseg - 1; pass B runs
// segments 1 .. nseg - 1 from those entries, with outputs.  Each pass is
// one round of workgroups, each walking at most ncs chunks instead of the
// whole sequence.
//
// A workgroup of a segment launch either runs segment s with outputs
// (workgroups 0 .. nout - 1: tile, head, segment, batch row, fastest first)
// or forms segment s's transition (the rest: tile of the transition's
// columns, head, segment, batch row).  The transition's columns are the
// local part (the DV value columns, from a zero entry) and then the columns
// of Phi_s: DK columns from the entry S = e_j, M = 0, and with momentum DK
// more from S = 0, M = e_j.
struct SegArgs {
    int ncs;              // chunks per segment (the last may have fewer)
    int ncs0;             // chunks of segment 0 (at most ncs)
    int nseg;
    int out_s0, out_ns;   // the segments run with outputs
    unsigned nout;        // workgroups of those segments
    int tr_s0, tr_ns;     // the segments whose transitions are formed
    int ncol;             // columns of a transition: DV + DK (no momentum) or DV + 2 DK
    int heads8;           // B H is a multiple of 8 (the combine's block order)
    float* Sx;            // entry states [B][nseg][H][DK][DV] (segment 0: the caller's)
    float* Mx;
    float* ES;            // exit states of the transitions [B][tr_ns][H][DK][ncol]
    float* EM;
};

// MOM = false is the momentum-free case mu = 0 (the gated delta rule): then
// b = 0 and mubar = 0, so the momentum never feeds the memory, and the
// final momentum is the last token's own write, -eta_T k_T vt_T^T (the last
// chunk's update with the weights eta m_n, which are zero but on its last
// row); the compute waves skip every product with M.
// TRANS (segment scan only): this workgroup forms a transition.
template <int DK, int DV, bool MOM, bool SAVE, bool SEG, bool TRANS>
__device__ __forceinline__ void fused_body(
    char* smem, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const float* __restrict__ ctab, const float* S0,
    const float* M0, __bf16* __restrict__ O, __bf16* __restrict__ Vto, float* ST, float* MT,
    int T, int H, int NC, int xcd_groups, const SegArgs& sg)
{
    static_assert(!(SEG && SAVE) && (SEG || !TRANS), "segment roles");
    using E = __bf16;
    using MM = Mma<E>;
    using L = FusedLayout<DK>;
    using LK = typename L::LK;
    using LC = typename L::LC;
    using CTb = ChunkTables;
    constexpr int TV = 64;                  // value columns per workgroup
    constexpr int NTILE = DV / TV;
    constexpr int RT = DK / 16;             // state row tiles
    constexpr int SK = DK / 32;             // 16x16x32 k-steps over d
    static_assert(DV % TV == 0, "value tile");

    // coefficient tables of chunk c: set c & 1
    auto tables = [&](int c) {
        return reinterpret_cast<float*>(smem + L::OFF_TB + (c & 1) * L::TB_BYTES);
    };
    auto kbuf = [&](int c) { return smem + L::OFF_K + (c % 3) * LK::BYTES; };
    auto qbuf = [&](int c) { return smem + L::OFF_Q + (c % 3) * LK::BYTES; };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;

    unsigned bid = blockIdx.x;
    if (xcd_groups > 0) bid = (bid % 8u) * (unsigned)xcd_groups + bid / 8u;
    // this workgroup's chunks c0 .. c0 + NCL - 1 (local index c: chunk c0 + c)
    int tile, h, b, seg = 0, c0 = 0, NCL = NC;
    constexpr bool trans = TRANS;           // forms a transition: no outputs
    if constexpr (!SEG) {
        tile = (int)(bid % NTILE);
        const int bh0 = (int)(bid / NTILE);
        h = bh0 % H;
        b = bh0 / H;
    } else {
        constexpr int NTALL = NTILE + (MOM ? 2 : 1) * (DK / TV);
        unsigned r;
        if constexpr (!TRANS) {
            tile = (int)(bid % NTILE);
            r = bid / NTILE;
            h = (int)(r % (unsigned)H);
            r /= (unsigned)H;
            seg = sg.out_s0 + (int)(r % (unsigned)sg.out_ns);
            b = (int)(r / (unsigned)sg.out_ns);
        } else {
            const unsigned i = bid - sg.nout;
            tile = (int)(i % NTALL);
            r = i / NTALL;
            h = (int)(r % (unsigned)H);
            r /= (unsigned)H;
            seg = sg.tr_s0 + (int)(r % (unsigned)sg.tr_ns);
            b = (int)(r / (unsigned)sg.tr_ns);
        }
        c0 = seg == 0 ? 0 : sg.ncs0 + (seg - 1) * sg.ncs;
        NCL = seg == 0 ? sg.ncs0 : min(sg.ncs, NC - c0);
    }
    const int bh = b * H + h;
    // the V tile the helpers stage (a transition's identity columns have no
    // V; they stage tile 0, which the compute waves then ignore)
    const int vtile = tile < NTILE ? tile : 0;
    // token index of row 0 of local chunk c of this head (rows are H tokens apart)
    auto tok_base = [&](int c) { return ((size_t)b * T + (size_t)(c0 + c) * CH) * H + h; };
    auto chunk_rows = [&](int c) { return min(CH, T - (c0 + c) * CH); };

    if (wave >= 4) {
        // =================== helper wavefronts ===================
        // Helper W builds row block W of T and row block X = 3 - W of A (five
        // 16x16 Gram tiles for every helper), from the K and Q tiles that all
        // four helpers' direct loads bring to LDS a chunk ahead.
        const int hw = wave - 4;
        const unsigned v_lane = LC::lane_offset((unsigned)(H * DV), lane);
        // 16x16 product X Y from acc(X^T) and acc(Y), where acc(Z) is the
        // accumulator layout (lane (l16, g), element r = Z[4 g + r][l16]): the
        // A operand of a 16x16x16 step is then acc(X^T) and the B operand
        // acc(Y), both straight from registers (operands rounded to bf16)
        auto prod = [](const f32x4& XT, const f32x4& YB) {
            return mma16(to_bf4(XT), to_bf4(YB), zero4());
        };
        // K and Q rows reach LDS by direct loads.  A K/Q tile is NWIN windows
        // of 1 KB; helper W takes windows W, W + 4, ...  Lane l of window w
        // fills tile bytes 1024 w + 16 l, which are one 16-byte slot of one
        // row of the padded, XOR-permuted layout, so it reads the logical
        // chunk stored in that slot (a slot past a row's data is padding: it
        // reads the row's first chunk and is never read back).  Rows past a
        // partial last chunk read its last row: their Gram entries reach only
        // the Vt and O rows past its end, which no output and no state update
        // uses (the coefficient rows and state weights vanish there).
        constexpr int NWIN = LK::BYTES / 1024;
        constexpr int NWH = (NWIN + 3) / 4;
        static_assert(LK::BYTES % 1024 == 0, "whole windows");
        const unsigned rowbytes = (unsigned)(H * DK) * 2u;
        struct KQLane {
            unsigned off[NWH];   // source byte offset of the lane's slot in a whole chunk
            int row[NWH];        // its row
        };
        auto kq_lane = [&](auto wc) {
            constexpr int W = decltype(wc)::value;
            KQLane kl;
#pragma unroll
            for (int u = 0; u < NWH; ++u) {
                const int o = 1024 * (W + 4 * u) + 16 * lane;
                const int row = min(o / LK::STRIDE, CH - 1);
                const int p = (o - row * LK::STRIDE) / 16;
                const int qc = p < DK / 8 ? p ^ ((row >> 2) & 3) : 0;
                kl.row[u] = row;
                kl.off[u] = (unsigned)row * rowbytes + 16u * (unsigned)qc;
            }
            return kl;
        };
        // direct loads of chunk c's rows of K or Q (base) into tile dst
        auto load_kq = [&](auto wc, const KQLane& kl, const E* base, int c, char* dst) {
            constexpr int W = decltype(wc)::value;
            const char* src = reinterpret_cast<const char*>(base + tok_base(c) * DK);
            const int n = chunk_rows(c);
            unsigned o[NWH];
#pragma unroll
            for (int u = 0; u < NWH; ++u) o[u] = kl.off[u];
            if (n < CH) {
#pragma unroll
                for (int u = 0; u < NWH; ++u)
                    o[u] = kl.off[u] - (unsigned)max(kl.row[u] - (n - 1), 0) * rowbytes;
            }
#pragma unroll
            for (int u = 0; u < NWH; ++u)
                if (W + 4 * u < NWIN) direct_load16(src + o[u], dst + 1024 * (W + 4 * u));
        };
        // direct loads of chunk c's V tile and coefficient rows into buffer B
        auto load_v = [&](int c, char* B) {
            const int n = chunk_rows(c);
            LC::load(B + L::OFF_V, v + tok_base(c) * DV + vtile * TV, (unsigned)(H * DV), v_lane,
                     n, hw, lane);
            const float* src = ctab + ((size_t)bh * NC + c0 + c) * CTb::FLOATS + CTb::VEC;
            if (hw == 0 || (hw == 1 && lane < 32))
                direct_load16(src + 4 * (64 * hw + lane), B + L::OFF_VEC + 1024 * hw);
        };
        // direct loads of chunk c's tables into its table set: 5 pieces of
        // 1 KB, helper h takes pieces h and h + 4
        auto load_tables = [&](int c) {
            const float* src = ctab + ((size_t)bh * NC + c0 + c) * CTb::FLOATS;
            char* dst = reinterpret_cast<char*>(tables(c));
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int piece = hw + 4 * u;
                if (piece < CTb::LDS_FLOATS / 256)
                    direct_load16(src + 256 * piece + 4 * lane, dst + 1024 * piece);
            }
        };

        // Elementwise factors of helper W's Gram tiles, from chunk tables tb.
        // Lane layout of the tiles: (row 16 x + l16, columns 16 J + 4 lg + r).
        //   mL[J]: -N_{W,J} = mL[J] o G_{W,J} (J < W): -alpha_i eta_j gamma_{i-1,j}
        //   mT, mB: N_{W,W} in both accumulator layouts (zero on and above the
        //           diagonal): alpha_i eta_j gamma_{i-1,j}; mB is N_{W,W}'s own
        //           layout (row 16 W + 4 lg + r, column 16 W + l16)
        //   mA[J]: A_{X,J} = mA[J] o (Q K^T)_{X,J} (J <= X): eta_j gamma_{i,j}
        struct Mult {
            f32x4 mL[3], mT, mB, mA[4];
        };
        // the lane's table offsets and 0/1 masks, the same every chunk
        struct MultLane {
            int oP;          // row iL - 1 (iL itself on the block's first row)
            int oGdT;        // GD row iL - 1 (clamped), columns 4 lg ..
            int oGdB[4];     // GD row 16 W + 4 lg + r - 1, column l16
            int oGdA;        // GD row 16 X + l16, columns 4 lg .. (the zeros past its stored part)
            float z0;        // 1 on the block's first row
            f32x4 fT, fB;    // strictly below the diagonal in either layout
            f32x4 id;        // the identity in the accumulator layout
        };
        auto mult_lane = [&](auto wc) {
            constexpr int W = decltype(wc)::value;
            MultLane ml;
            const int iL = 16 * W + l16;
            ml.oP = l16 > 0 ? iL - 1 : iL;
            // entries read past a row's stored part are masked below (fT, fB)
            // and finite; A's diagonal block has no mask, so its lanes past
            // the stored part read the zeros
            ml.oGdT = CTb::GD + gd_row(16 * W + (l16 > 0 ? l16 - 1 : 0)) + 4 * lg;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * W + 4 * lg + r - 1;      // -1 (W = 0): masked
                ml.oGdB[r] = row < 0 ? CTb::GD_ZERO : CTb::GD + gd_row(row) + l16;
            }
            const int iA = 16 * (3 - W) + l16;
            ml.oGdA = 4 * lg < gd_len(iA) ? CTb::GD + gd_row(iA) + 4 * lg : CTb::GD_ZERO;
            ml.z0 = l16 == 0 ? 1.f : 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 4 * lg + r;
                ml.fT[r] = j < l16 ? 1.f : 0.f;
                ml.fB[r] = l16 < j ? 1.f : 0.f;
                ml.id[r] = j == l16 ? 1.f : 0.f;
            }
            return ml;
        };
        auto multipliers = [&](auto wc, const float* tb, const MultLane& ml) {
            constexpr int W = decltype(wc)::value;
            constexpr int X = 3 - W;
            Mult m;
            const int iL = 16 * W + l16;
            const float aiL = tb[CTb::ALPHA + iL];
            const float raP = tb[CTb::RA + ml.oP], rgP = tb[CTb::RG + ml.oP];
            // gamma_{i-1,j} = raP gb + rgP mb, and gb itself on the first row;
            // -alpha_i folded into the two row factors (the tables carry eta_j)
            const float raZ = raP + ml.z0 * (1.f - raP), rgZ = rgP - ml.z0 * rgP;
            const float cL = -aiL * raZ, dL = -aiL * rgZ;
#pragma unroll
            for (int J = 0; J < W; ++J) {
                const f32x4 gb = *reinterpret_cast<const f32x4*>(tb + CTb::GB + 64 * (W - 1) + 16 * J + 4 * lg);
                const f32x4 mb = *reinterpret_cast<const f32x4*>(tb + CTb::MB + 64 * (W - 1) + 16 * J + 4 * lg);
                m.mL[J] = cL * gb + dL * mb;
            }
            const f32x4 gdT = *reinterpret_cast<const f32x4*>(tb + ml.oGdT);
            const f32x4 aD = *reinterpret_cast<const f32x4*>(tb + CTb::ALPHA + 16 * W + 4 * lg);
            f32x4 gdB;
#pragma unroll
            for (int r = 0; r < 4; ++r) gdB[r] = tb[ml.oGdB[r]];
            m.mT = ml.fT * (aiL * gdT);
            m.mB = ml.fB * (aD * gdB);
            const int iA = 16 * X + l16;
            const float ra = tb[CTb::RA + iA], rg = tb[CTb::RG + iA];
#pragma unroll
            for (int J = 0; J < X; ++J) {
                const f32x4 gb = *reinterpret_cast<const f32x4*>(tb + CTb::GB + 64 * (X - 1) + 16 * J + 4 * lg);
                const f32x4 mb = *reinterpret_cast<const f32x4*>(tb + CTb::MB + 64 * (X - 1) + 16 * J + 4 * lg);
                m.mA[J] = ra * gb + rg * mb;
            }
            m.mA[X] = *reinterpret_cast<const f32x4*>(tb + ml.oGdA);
            return m;
        };

        // One row block x of T or A into its fragment slots: pairs
        // (J, J + 1) as one 16-byte store, lone blocks as 8 bytes
        auto store_block_row = [&](auto xc, char* area, const bf16x4* f) {
            constexpr int x = decltype(xc)::value;
#pragma unroll
            for (int J = 0; J <= x; ++J) {
                const FragSlot sl = frag_slot(x, J);
                if (sl.stride == 8)
                    *reinterpret_cast<bf16x4*>(area + sl.off + 8 * lane) = f[J];
                else if ((J & 1) == 0)
                    *reinterpret_cast<bf16x8*>(area + sl.off + 16 * lane) = cat8(f[J], f[J + 1]);
            }
        };

        // Row block W of L (-N_{W,J}, J < W, and D_W) into T, row block X
        // of A into A, for the chunk whose K and Q tiles are Kt and Qt; W is
        // this helper's index, a compile-time constant in each copy.
        auto prepare = [&](auto wc, char* B, const char* Kt, const char* Qt, const Mult& m,
                           const f32x4& Id) {
            constexpr int W = decltype(wc)::value;
            constexpr int X = 3 - W;
            // K blocks 0 .. JN are read (a transition forms no A: it has no outputs)
            constexpr int JN = TRANS ? W : W > X ? W : X;
            // ---- Gram tiles, transposed (lane: row 16 x + l16, columns 16 J + 4 lg + r)
            f32x4 Gt[W + 1], At[X + 1];
#pragma unroll
            for (int J = 0; J <= W; ++J) Gt[J] = zero4();
#pragma unroll
            for (int J = 0; J <= X; ++J) At[J] = zero4();
#pragma unroll
            for (int s = 0; s < SK; ++s) {
                MM::frag aK[JN + 1];
#pragma unroll
                for (int J = 0; J <= JN; ++J)
                    aK[J] = *reinterpret_cast<const MM::frag*>(Kt + LK::chunk(16 * J + l16, 4 * s + lg));
#pragma unroll
                for (int J = 0; J <= W; ++J) Gt[J] = MM::mma(aK[J], aK[W], Gt[J]);
                if constexpr (!TRANS) {
                    const MM::frag aQ =
                        *reinterpret_cast<const MM::frag*>(Qt + LK::chunk(16 * X + l16, 4 * s + lg));
#pragma unroll
                    for (int J = 0; J <= X; ++J) At[J] = MM::mma(aK[J], aQ, At[J]);
                }
            }
            // N_WW in both accumulator layouts from the symmetric Gram tile:
            // NT = acc(N^T) (lane: row l16, cols 4 lg + r), NB = acc(N)
            const f32x4 NT = m.mT * Gt[W], NB = m.mB * Gt[W];
            // D_W = (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0),
            // formed transposed: D^T = (I + N8^T)(I + N4^T) P1^T
            const f32x4 N2B = prod(NT, NB), N2T = prod(NB, NT);
            const f32x4 N4B = prod(N2T, N2B), N4T = prod(N2B, N2T);
            const f32x4 N8B = prod(N4T, N4B);
            const f32x4 P1T = Id - NT + N2T - prod(N2B, NT);
            const f32x4 QT = P1T + prod(N4B, P1T);
            const f32x4 DT = QT + prod(N8B, QT);
            // ---- stores
            bf16x4 tW[W + 1], aX[X + 1];
#pragma unroll
            for (int J = 0; J < W; ++J) tW[J] = to_bf4(m.mL[J] * Gt[J]);
            tW[W] = to_bf4(DT);
            store_block_row(IConst<W>{}, B + L::OFF_T, tW);
            if constexpr (!TRANS) {
#pragma unroll
                for (int J = 0; J <= X; ++J) aX[J] = to_bf4(m.mA[J] * At[J]);
                store_block_row(IConst<X>{}, B + L::OFF_A, aX);
            }
        };

        // The pipeline: in round c (c = -1 .. NC - 1) chunk nx = c + 1 is
        // prepared into operand buffer nx & 1 while the compute wavefronts
        // scan chunk c.  At the start of the round the K and Q tiles and the
        // tables of nx are in LDS (loaded in round c - 1).  The round issues
        // the direct loads of the tables, K and Q rows of nx + 1 and of the V
        // tile and coefficient rows of nx, builds nx's T and A, and waits for
        // its loads before the barrier: everything the next round reads has
        // then landed.
        auto run = [&](auto wc) {
            const MultLane ml = mult_lane(wc);
            const KQLane kl = kq_lane(wc);
            auto round = [&](int c, auto par) {      // par: parity of nx
                constexpr int P = decltype(par)::value;
                const int nx = c + 1;
                char* B = smem + P * L::BUF;
                if (nx < NCL) {
                    if (nx + 1 < NCL) {
                        load_tables(nx + 1);
                        load_kq(wc, kl, k, nx + 1, kbuf(nx + 1));
                        if constexpr (!TRANS) load_kq(wc, kl, q, nx + 1, qbuf(nx + 1));
                    }
                    load_v(nx, B);
                    const Mult m = multipliers(wc, tables(nx), ml);
                    prepare(wc, B, kbuf(nx), qbuf(nx), m, ml.id);
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
                lds_barrier();   // B0: chunk nx ready
            };
            // the K, Q tiles and tables of chunk 0
            load_kq(wc, kl, k, 0, kbuf(0));
            if constexpr (!TRANS) load_kq(wc, kl, q, 0, qbuf(0));
            load_tables(0);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();       // chunk 0's K, Q tiles and tables visible
            for (int c = -1; c < NCL; c += 2) {
                round(c, IConst<0>{});
                if (c + 1 < NCL) round(c + 1, IConst<1>{});
            }
        };
        switch (hw) {
        case 0: run(IConst<0>{}); break;
        case 1: run(IConst<1>{}); break;
        case 2: run(IConst<2>{}); break;
        default: run(IConst<3>{}); break;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }

    // =================== compute wavefronts ===================
    const int wl = 16 * wave + l16;            // this lane's column inside the tile
    const int col = tile * TV + wl;            // ... inside the head (or the transition)
    f32x4 Sa[RT], Ma[RT];                      // slot (rt, lg, r): row phys_row(16 rt + 4 lg + r)
    // entry and exit states: rows ld floats apart from a per-workgroup base
    // (the state of head bh, or of segment seg of it)
    const size_t sbase = (size_t)bh * DK * DV;
    const float* s0p = S0 ? S0 + sbase : nullptr;
    const float* m0p = M0 ? M0 + sbase : nullptr;
    float* stp = ST ? ST + sbase : nullptr;
    float* mtp = MT ? MT + sbase : nullptr;
    int ld = DV;
    if constexpr (SEG) {
        auto seg_state = [&](float* X, int s) {
            return X + (((size_t)b * sg.nseg + s) * H + h) * DK * DV;
        };
        if (trans) {
            const size_t tb = (((size_t)b * sg.tr_ns + (seg - sg.tr_s0)) * H + h) * DK * sg.ncol;
            s0p = m0p = nullptr;
            stp = sg.ES + tb;
            mtp = MOM ? sg.EM + tb : nullptr;
            ld = sg.ncol;
        } else {
            if (seg > 0) {
                s0p = seg_state(sg.Sx, seg);
                m0p = seg_state(sg.Mx, seg);
            }
            if (seg < sg.nseg - 1) {
                // segment 0 hands its exit state to segment 1; the others'
                // exits are already known
                stp = seg == 0 ? seg_state(sg.Sx, 1) : nullptr;
                mtp = seg == 0 && MOM ? seg_state(sg.Mx, 1) : nullptr;
            }
        }
    }
    auto load_state = [&](f32x4* X, const float* src) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                X[rt][r] = src ? src[(size_t)phys_row(16 * rt + 4 * lg + r) * ld + col] : 0.f;
    };
    if constexpr (SEG) {
        if (s0p) load_state(Sa, s0p); else load_state(Sa, nullptr);
        if (MOM && m0p) load_state(Ma, m0p); else load_state(Ma, nullptr);
    } else {
        auto load0 = [&](f32x4* X, const float* src) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    X[rt][r] = src ? src[sbase + (size_t)phys_row(16 * rt + 4 * lg + r) * DV + col] : 0.f;
        };
        if (S0) load0(Sa, S0); else load0(Sa, nullptr);
        if (MOM && M0) load0(Ma, M0); else load0(Ma, nullptr);
    }
    // a transition's identity columns: column j of Phi starts from S = e_j
    // (the first DK) or M = e_j (the next DK)
    const bool phi = SEG && trans && tile >= NTILE;
    if (phi) {
        const int j = (tile - NTILE) * TV + wl;
        f32x4* X = MOM && j >= DK ? Ma : Sa;
        const int jj = j % DK;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) X[rt][r] = phys_row(16 * rt + 4 * lg + r) == jj ? 1.f : 0.f;
    }

    // per-lane LDS offsets, the same every chunk
    // row 16 x + l16, d-chunk lg: rows 16 apart share the swizzle, so the
    // four row blocks are one lane offset plus a constant
    const int kq0 = LK::chunk(l16, lg);
    auto kq_base = [&](int x) { return kq0 + x * LK::J16; };
    // transposing reads: lane 4 j + m of a 16-lane group reads row base + j,
    // 4 columns starting at 4 m of the wanted column block
    const int trj = l16 >> 2, trm = l16 & 3;
    // K rows 4 lg + j (+ 16 J), columns d0 = phys_row(16 rt + 4 m) .. + 3,
    // with d0 = 32 (rt >> 1) + 8 m + 4 (rt & 1): the d-chunk is
    // 4 (rt >> 1) + m, whose swizzle with key (row >> 2) & 3 = lg leaves
    // 4 (rt >> 1) alone, so every rt is one lane offset plus a constant
    // (instruction immediates instead of an address add per read)
    const int ktr0 = LK::chunk(4 * lg + trj, trm);
    auto ktr_base = [&](int rt) { return ktr0 + 64 * (rt >> 1) + 8 * (rt & 1); };
    constexpr int KJ = LK::J16;                // 16 K rows further
    const int vc = 16 * wave + 4 * trm;
    const int vtr_base = LC::chunk(4 * lg + trj, vc >> 3) + 2 * (vc & 7);
    constexpr int VJ = 16 * CH * 2 + (16 / LC::G) * LC::PAD;   // 16 V rows further
    const unsigned ostride = (unsigned)(H * DV);
    E* const Ocol = O + ((size_t)b * T * H + h) * DV + tile * TV + 16 * wave + 4 * lg;
    // SAVE: the residuals Vt of every token, [B, T, H, DV] like O (a backward
    // pass can then rebuild the states without the solve)
    E* const Vcol = SAVE ? Vto + ((size_t)b * T * H + h) * DV + tile * TV + 16 * wave + 4 * lg : nullptr;
    // the 16 x 16 identity as a B fragment of mma16: B[4 lg + j][l16] = (4 lg + j == l16)
    bf16x4 eye;
#pragma unroll
    for (int j = 0; j < 4; ++j) eye[j] = static_cast<__bf16>(4 * lg + j == l16 ? 1.f : 0.f);

    lds_barrier();   // chunk 0's tables in LDS
    lds_barrier();   // B0: chunk 0 ready
    for (int c = 0; c < NCL; ++c) {
        const int t0 = (c0 + c) * CH;
        const int n = min(CH, T - t0);
        const char* B = smem + (c & 1) * L::BUF;
        const char* Kb = kbuf(c);
        const char* Qb = qbuf(c);
        const char* Vb = B + L::OFF_V;
        const char* Tb = B + L::OFF_T;
        const char* Ab = B + L::OFF_A;
        const float* vec = reinterpret_cast<const float*>(B + L::OFF_VEC);

        // The chunk's products on the state and the substitution are each
        // scheduled by the compiler's single-wave small-GEMM interleaving
        // (LDS reads hoisted ahead of the MFMAs that take them, vector work
        // placed between independent MFMAs): measured 4-5% faster per call
        // than its default schedule at 1.3B-like, 400M-like and 16K-context
        // shapes, bit-identical.
        __builtin_amdgcn_iglp_opt(1);
        // (1) X = K [S | M]
        f32x4 R[4];
        {
            f32x4 xs[4], xm[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) xs[ct] = xm[ct] = zero4();
#pragma unroll
            for (int s = 0; s < SK; ++s) {
                const auto bS = MM::from_acc(Sa, s);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const auto aK = *reinterpret_cast<const MM::frag*>(Kb + kq_base(ct) + 64 * s);
                    xs[ct] = MM::mma(aK, bS, xs[ct]);
                    if constexpr (MOM) xm[ct] = MM::mma(aK, MM::from_acc(Ma, s), xm[ct]);
                }
            }
            // (2) R = V - Diag(abar) K S0 + Diag(alpha b^-) K M0, rows 16 ct + 4 lg + r
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int p0 = 16 * ct + 4 * lg;
                const f32x4 ab = *reinterpret_cast<const f32x4*>(vec + V_ABAR * CH + p0);
                const f32x4 ab1 = *reinterpret_cast<const f32x4*>(vec + V_AB1 * CH + p0);
                const bf16x4 vv = lds_read_tr4(Vb + vtr_base + ct * VJ);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    R[ct][r] = (phi ? 0.f : static_cast<float>(vv[r])) - ab[r] * xs[ct][r];
                    if constexpr (MOM) R[ct][r] += ab1[r] * xm[ct][r];
                }
            }
        }
        // (3) O^T = S0^T Q^T Diag(abar) - M0^T Q^T Diag(b) + Vt^T A^T, its
        //     entry-state part now (it needs nothing the helpers produce);
        //     lane: output row 16 ct + l16, columns 4 lg .. + 3 of this
        //     wavefront's 16
        // (a transition has no outputs: its workgroups skip the Q and A
        // products and the stores)
        const bool outputs = !(SEG && trans);
        f32x4 Ot[4];
        if (outputs) {
            f32x4 ys[4], ym[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) ys[ct] = ym[ct] = zero4();
#pragma unroll
            for (int s = 0; s < SK; ++s) {
                const auto bS = MM::from_acc(Sa, s);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const auto aQ = *reinterpret_cast<const MM::frag*>(Qb + kq_base(ct) + 64 * s);
                    ys[ct] = MM::mma(bS, aQ, ys[ct]);
                    if constexpr (MOM) ym[ct] = MM::mma(MM::from_acc(Ma, s), aQ, ym[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const float ab = vec[V_ABAR * CH + 16 * ct + l16];
                Ot[ct] = ab * ys[ct];
                if constexpr (MOM) Ot[ct] -= vec[V_B * CH + 16 * ct + l16] * ym[ct];
            }
        }

        __builtin_amdgcn_iglp_opt(1);
        // (4) Vt = L^{-1} R by block substitution; T's blocks: D on the
        //     diagonal, -N below it (pairs read as one 16-byte access)
        f32x4 Vt[4];
        {
            const bf16x8 t10 = *reinterpret_cast<const bf16x8*>(Tb + frag_slot(1, 0).off + 16 * lane);
            const bf16x8 t20 = *reinterpret_cast<const bf16x8*>(Tb + frag_slot(2, 0).off + 16 * lane);
            const bf16x8 t30 = *reinterpret_cast<const bf16x8*>(Tb + frag_slot(3, 0).off + 16 * lane);
            const bf16x8 t32 = *reinterpret_cast<const bf16x8*>(Tb + frag_slot(3, 2).off + 16 * lane);
            const bf16x4 t00 = *reinterpret_cast<const bf16x4*>(Tb + frag_slot(0, 0).off + 8 * lane);
            const bf16x4 t22 = *reinterpret_cast<const bf16x4*>(Tb + frag_slot(2, 2).off + 8 * lane);
            const bf16x4 tb[4][4] = {{t00, t00, t00, t00},
                                     {lo4(t10), hi4(t10), t00, t00},
                                     {lo4(t20), hi4(t20), t22, t00},
                                     {lo4(t30), hi4(t30), lo4(t32), hi4(t32)}};
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                Vt[I] = mma16(tb[I][I], to_bf4(R[I]), zero4());
                const bf16x4 vI = to_bf4(Vt[I]);
#pragma unroll
                for (int I2 = I + 1; I2 < 4; ++I2) R[I2] = mma16(tb[I2][I], vI, R[I2]);
            }
        }

        // ... and its chunk-local part, over the blocks J <= ct of A's row
        //     tile ct; blocks 2 p and 2 p + 1 together make one 16x16x32 step
        //     (k = their 32 rows), a lone block a 16x16x32 step with zero
        //     upper half.  Every step of an accumulator's chain has the same
        //     shape: an MFMA that takes the result of an MFMA of another
        //     shape as its accumulator input, with no instruction between,
        //     has read a stale accumulator on gfx950 (the compiler inserts
        //     no wait there), and the 16x16x16 form is no faster here.
        if (outputs) {
            bf16x4 vb[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) vb[J] = to_bf4(Vt[J]);
            const bf16x4 zb = to_bf4(zero4());
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
                for (int p = 0; 2 * p <= ct; ++p) {
                    const FragSlot f = frag_slot(ct, 2 * p);
                    if (2 * p + 1 <= ct) {
                        const bf16x8 a01 = *reinterpret_cast<const bf16x8*>(Ab + f.off + 16 * lane);
                        Ot[ct] = MM::mma(cat8(vb[2 * p], vb[2 * p + 1]), a01, Ot[ct]);
                    } else {
                        const bf16x4 a0 = *reinterpret_cast<const bf16x4*>(Ab + f.off + 8 * lane);
                        Ot[ct] = MM::mma(cat8(vb[2 * p], zb), cat8(a0, zb), Ot[ct]);
                    }
                }
            }
        }
        if (outputs) {
            // One 16-byte store per lane per pair of row tiles: lane groups
            // lg and lg ^ 1 (lg = 2 x, 2 x + 1) swap halves of row tiles 2 p and
            // 2 p + 1 (permlane16_swap exchanges group 1 of its first operand
            // with group 0 of its second, and group 3 with group 2), after which
            // each lane holds 8 consecutive columns, 8 x .. 8 x + 7 of this
            // wave's 16, of row 16 (2 p + (lg & 1)) + l16.  Half the store
            // instructions of one 8-byte store per row tile.
            E* Ob = Ocol - 4 * lg + 8 * (lg >> 1) + (size_t)t0 * ostride;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                u32x2 ua = __builtin_bit_cast(u32x2, to_bf4(Ot[2 * p]));
                u32x2 ub = __builtin_bit_cast(u32x2, to_bf4(Ot[2 * p + 1]));
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const auto r = __builtin_amdgcn_permlane16_swap(ua[d], ub[d], false, false);
                    ua[d] = r[0];
                    ub[d] = r[1];
                }
                const int row = 16 * (2 * p + (lg & 1)) + l16;
                if (row < n)
                    *reinterpret_cast<u32x4*>(Ob + (unsigned)row * ostride) = u32x4{ua[0], ua[1], ub[0], ub[1]};
            }
        }
        if constexpr (SAVE) {
            // Vt[I] element r is row 16 I + 4 lg + r, column l16 of this wave's
            // 16.  One MFMA per block with the identity, Vt_I^T I, puts it in
            // O's layout (element r: row 16 I + l16, column 4 lg + r) with the
            // same bf16 values; then O's two 16-byte stores per lane.
            f32x4 Vtt[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) Vtt[I] = mma16(to_bf4(Vt[I]), eye, zero4());
            E* Vb = Vcol - 4 * lg + 8 * (lg >> 1) + (size_t)t0 * ostride;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                u32x2 ua = __builtin_bit_cast(u32x2, to_bf4(Vtt[2 * p]));
                u32x2 ub = __builtin_bit_cast(u32x2, to_bf4(Vtt[2 * p + 1]));
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const auto r = __builtin_amdgcn_permlane16_swap(ua[d], ub[d], false, false);
                    ua[d] = r[0];
                    ub[d] = r[1];
                }
                const int row = 16 * (2 * p + (lg & 1)) + l16;
                if (row < n)
                    *reinterpret_cast<u32x4*>(Vb + (unsigned)row * ostride) = u32x4{ua[0], ua[1], ub[0], ub[1]};
            }
        }

        // (5) S' = abar_n S0 - b_n M0 + K^T Diag(eta gamma_n) Vt,
        //     M' = mubar_n M0 - K^T Diag(eta mubar_n / mubar) Vt
        const float abn = vec[V_SCAL * CH + 0];
        const float bn = vec[V_SCAL * CH + 1];
        const float mbn = vec[V_SCAL * CH + 2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if constexpr (MOM) {
                Sa[rt] = abn * Sa[rt] - bn * Ma[rt];
                Ma[rt] = mbn * Ma[rt];
            } else {
                (void)bn, (void)mbn;
                Sa[rt] = abn * Sa[rt];
            }
        }

        // K^T fragments by transposing reads, two 16-row blocks of the chunk
        // per 16x16x32 step (k = chunk rows 32 p .. 32 p + 31).  The lane's
        // base address is fixed here, so that every read is that base plus an
        // instruction immediate (left to itself the compiler rebases on a
        // later block and pays an address add per read for the negative
        // offsets of the others).
        const int ktb = opaque((int)(Kb - smem) + ktr0);
        // the products with K^T; `with_m` also updates M
        auto update = [&](auto with_m) {
            constexpr bool WM = decltype(with_m)::value != 0;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                bf16x4 bS[2], bM[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int J = 2 * p + e;
                    const f32x4 ws = *reinterpret_cast<const f32x4*>(vec + V_WS * CH + 16 * J + 4 * lg);
                    const f32x4 wm = *reinterpret_cast<const f32x4*>(vec + V_WM * CH + 16 * J + 4 * lg);
                    bS[e] = to_bf4(ws * Vt[J]);
                    if constexpr (WM) bM[e] = to_bf4(-(wm * Vt[J]));
                }
                const auto bS8 = cat8(bS[0], bS[1]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const int off = ktr_base(rt) - ktr0;   // a constant
                    const auto aK = cat8(lds_read_tr4(smem + ktb + off + 2 * p * KJ),
                                         lds_read_tr4(smem + ktb + off + (2 * p + 1) * KJ));
                    Sa[rt] = MM::mma(aK, bS8, Sa[rt]);
                    if constexpr (WM) Ma[rt] = MM::mma(aK, cat8(bM[0], bM[1]), Ma[rt]);
                }
            }
        };
        if constexpr (MOM) {
            update(IConst<1>{});
        } else if ((SEG ? mtp != nullptr : MT != nullptr) && c == NCL - 1) {
            // without momentum M' is the last token's own write; it is
            // formed once, with the last chunk (M is zero before it)
            update(IConst<1>{});
        } else {
            update(IConst<0>{});
        }
        lds_barrier();   // B0: chunk c + 1 ready, this buffer free
    }

    auto store_state = [&](float* dst, const f32x4* X) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(size_t)phys_row(16 * rt + 4 * lg + r) * ld + col] = X[rt][r];
    };
    if constexpr (SEG) {
        if (stp) store_state(stp, Sa);
        if (mtp) store_state(mtp, Ma);
    } else {
        auto store0 = [&](float* dst, const f32x4* X) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[sbase + (size_t)phys_row(16 * rt + 4 * lg + r) * DV + col] = X[rt][r];
        };
        if (ST) store0(ST, Sa);
        if (MT) store0(MT, Ma);
    }
}

template <int DK, int DV, bool MOM, bool SAVE>
__global__ __launch_bounds__(2 * NT) void chunk_fwd_fused_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* __restrict__ ctab, const float* S0, const float* M0, __bf16* __restrict__ O,
    __bf16* __restrict__ Vto, float* ST, float* MT, int T, int H, int NC, int xcd_groups)
{
    __shared__ __align__(16) char smem[FusedLayout<DK>::BYTES];
    fused_body<DK, DV, MOM, SAVE, false, false>(smem, q, k, v, ctab, S0, M0, O, Vto, ST, MT, T,
                                                H, NC, xcd_groups, SegArgs{});
}

// One pass of the segment scan (see SegArgs): S0, M0, ST, MT are the
// caller's states, read by segment 0 and written by the last segment.
template <int DK, int DV, bool MOM>
__global__ __launch_bounds__(2 * NT) void chunk_fwd_seg_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* __restrict__ ctab, const float* S0, const float* M0, __bf16* __restrict__ O,
    float* ST, float* MT, int T, int H, int NC, int xcd_groups, SegArgs sg)
{
    __shared__ __align__(16) char smem[FusedLayout<DK>::BYTES];
    unsigned bid = blockIdx.x;
    if (xcd_groups > 0) bid = (bid % 8u) * (unsigned)xcd_groups + bid / 8u;
    if (bid < sg.nout)
        fused_body<DK, DV, MOM, false, true, false>(smem, q, k, v, ctab, S0, M0, O, nullptr, ST,
                                                    MT, T, H, NC, xcd_groups, sg);
    else
        fused_body<DK, DV, MOM, false, true, true>(smem, q, k, v, ctab, S0, M0, O, nullptr, ST,
                                                   MT, T, H, NC, xcd_groups, sg);
}

// ---------------------------------------------------------------------------
// The entry states of the segment scan's segments 2 .. nseg - 1, in order:
// [S; M] entering segment s + 1 is segment s's local exit [S; M] plus Phi_s
// times [S; M] entering segment s (without momentum, S alone: M never feeds
// the memory there).  One workgroup per (batch row, head, 16 value columns):
// the columns are independent; one wavefront per 16 rows of [S; M].
// Products on bf16 MFMA with both operands
// split into a bf16 head and a bf16 remainder (three products: the
// remainder times remainder term is below fp32 rounding), so the states
// carry about fp32 accuracy across the segments.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool MOM>
__global__ __launch_bounds__((MOM ? 2 * DK : DK) * 4) void seg_combine_kernel(SegArgs sg, int H)
{
    using MM = Mma<__bf16>;
    constexpr int R2 = MOM ? 2 * DK : DK;   // rows of the carried pair
    constexpr int NTH = R2 * 4;             // one wavefront per 16-row output tile
    constexpr int KS = R2 / 32;             // 16x16x32 k-steps
    constexpr int CB = DV / 16;             // column blocks per head
    __shared__ float X[R2][17];             // the entry state, this block's 16 columns

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
    const int wave = tid >> 6;
    // The column blocks of a head read the same maps: with the heads a
    // multiple of 8, block i runs on XCD i mod 8, so blocks 8 (cb + CB j) + x
    // (all cb) of head 8 j + x share that XCD's L2
    int cb, bh;
    if (sg.heads8) {
        const unsigned x = blockIdx.x % 8u, r = blockIdx.x / 8u;
        cb = (int)(r % CB);
        bh = (int)(8u * (r / CB) + x);
    } else {
        cb = (int)(blockIdx.x % CB);
        bh = (int)(blockIdx.x / CB);
    }
    const int h = bh % H, b = bh / H;
    auto state_row = [&](int s, int row) {   // row of [S; M] entering segment s
        float* base = row < DK ? sg.Sx : sg.Mx;
        return base + ((((size_t)b * sg.nseg + s) * H + h) * DK + row % DK) * DV + 16 * cb;
    };
    for (int i = tid; i < R2 * 16; i += NTH) X[i / 16][i % 16] = state_row(sg.tr_s0, i / 16)[i % 16];
    __syncthreads();
    auto split = [](const float* x, MM::frag& hi, MM::frag& lo) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            hi[j] = static_cast<__bf16>(x[j]);
            lo[j] = static_cast<__bf16>(x[j] - static_cast<float>(hi[j]));
        }
    };
    for (int st = 0; st < sg.tr_ns; ++st) {
        const size_t tb = (((size_t)b * sg.tr_ns + st) * H + h) * DK * sg.ncol;
        auto erow = [&](int row) { return (row < DK ? sg.ES : sg.EM) + tb + (size_t)(row % DK) * sg.ncol; };
        // the step's A fragments (this wavefront's 16 rows of Phi) and its
        // local exit, all loaded before the products so that their latency
        // is paid once
        const float* arow = erow(16 * wave + l16) + DV + 8 * lg;
        f32x4 a0[KS], a1[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            a0[ks] = *reinterpret_cast<const f32x4*>(arow + 32 * ks);
            a1[ks] = *reinterpret_cast<const f32x4*>(arow + 32 * ks + 4);
        }
        f32x4 acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = erow(16 * wave + 4 * lg + r)[16 * cb + l16];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float xb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) xb[j] = X[32 * ks + 8 * lg + j][l16];
            MM::frag bh8, bl8, ah8, al8;
            split(xb, bh8, bl8);
            const float xa[8] = {a0[ks][0], a0[ks][1], a0[ks][2], a0[ks][3],
                                 a1[ks][0], a1[ks][1], a1[ks][2], a1[ks][3]};
            split(xa, ah8, al8);
            acc = MM::mma(ah8, bh8, acc);
            acc = MM::mma(ah8, bl8, acc);
            acc = MM::mma(al8, bh8, acc);
        }
        __syncthreads();   // every read of X is done
        const int s_next = sg.tr_s0 + st + 1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * wave + 4 * lg + r;
            X[row][l16] = acc[r];
            state_row(s_next, row)[l16] = acc[r];
        }
        __syncthreads();
    }
}

template <int DK, int DV>
static hipError_t launch_fused_t(const void* q, const void* k, const void* v, const float* alpha,
                                 const float* mu, const float* eta, const float* beta,
                                 const float* S0, const float* M0, void* O, void* Vto, float* ST,
                                 float* MT, int B, int T, int H, void* workspace,
                                 hipStream_t stream)
{
    const int NC = (T + CH - 1) / CH;
    float* ctab = static_cast<float*>(workspace);
    const unsigned nhg = (unsigned)((H + COEF_HEADS - 1) / COEF_HEADS);   // head groups
    hipLaunchKernelGGL(chunk_coef_kernel, dim3((unsigned)B * nhg * (unsigned)NC),
                       dim3(COEF_HEADS * 64), 0, stream, alpha, mu, eta, beta, ctab, T, H, NC,
                       nhg);
    const size_t nblk = (size_t)B * H * (DV / 64);
    const int xcd_groups = nblk % 8 == 0 ? (int)(nblk / 8) : 0;
    // mu = NULL: mu = 0, the momentum-free kernel
    // Vto != NULL: the variant that also stores the residuals
    auto kern = mu ? (Vto ? chunk_fwd_fused_kernel<DK, DV, true, true>
                          : chunk_fwd_fused_kernel<DK, DV, true, false>)
                   : (Vto ? chunk_fwd_fused_kernel<DK, DV, false, true>
                          : chunk_fwd_fused_kernel<DK, DV, false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(2 * NT), 0, stream,
                       static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                       static_cast<const __bf16*>(v), ctab, S0, M0, static_cast<__bf16*>(O),
                       static_cast<__bf16*>(Vto), ST, MT, T, H, NC, xcd_groups);
    return hipGetLastError();
}

// The whole bf16 forward for T >= 1: the coefficient kernel, then the fused
// kernel.  `workspace` holds chunk_fused_workspace_bytes(B * H * ceil(T / 64)).
hipError_t launch_chunk_fused(const void* q, const void* k, const void* v, const float* alpha,
                              const float* mu, const float* eta, const float* beta,
                              const float* S0, const float* M0, void* O, void* Vto, float* ST,
                              float* MT, int B, int T, int H, int Dk, int Dv, void* workspace,
                              hipStream_t stream)
{
    if (Dk == 128 && Dv == 128)
        return launch_fused_t<128, 128>(q, k, v, alpha, mu, eta, beta, S0, M0, O, Vto, ST, MT, B, T,
                                        H, workspace, stream);
    if (Dk == 128 && Dv == 64)
        return launch_fused_t<128, 64>(q, k, v, alpha, mu, eta, beta, S0, M0, O, Vto, ST, MT, B, T, H,
                                       workspace, stream);
    if (Dk == 64 && Dv == 128)
        return launch_fused_t<64, 128>(q, k, v, alpha, mu, eta, beta, S0, M0, O, Vto, ST, MT, B, T, H,
                                       workspace, stream);
    return launch_fused_t<64, 64>(q, k, v, alpha, mu, eta, beta, S0, M0, O, Vto, ST, MT, B, T, H,
                                  workspace, stream);
}

// ---------------------------------------------------------------------------
// Segment scan, host side.
// ---------------------------------------------------------------------------
// Workgroups one pass may take and still run as a single round: one per
// compute unit (each takes 140 KB of LDS), on a 256-CU MI355X.
constexpr int SEG_ROUND = 256;

// The number of segments for this shape (0: the segment scan does not
// apply).  Both passes must fit one round: pass A has the heads' tiles of
// segment 0 and the transitions of nseg - 2 segments, pass B the tiles of
// nseg - 1 segments.  A pass then walks ceil(NC / nseg) chunks, so the call
// walks 2 ceil(NC / nseg) in sequence against NC for the column tiles: three
// or more segments, each of at least min_ncs chunks.
int chunk_seg_count(int B, int T, int H, int Dk, int Dv, bool mom, int min_ncs)
{
    if (B <= 0 || T <= 0 || H <= 0) return 0;
    const long heads = (long)B * H;
    const long ntile = Dv / 64, ntall = ntile + (mom ? 2 : 1) * (Dk / 64);
    const long nc = ((long)T + CH - 1) / CH;
    int best = 0;
    for (int n = 3; n <= 64; ++n) {
        const long ncs = (nc + n - 1) / n;
        if (ncs < min_ncs || (n - 1) * ncs >= nc) break;
        if (heads * ntile + (n - 2) * heads * ntall > SEG_ROUND) break;
        if ((n - 1) * heads * ntile > SEG_ROUND) break;
        best = n;
    }
    return best;
}

namespace {
// Segment lengths: segment 0 runs in pass A beside the transitions of the
// middle segments, which form no outputs (no A, no Q products, no stores) and
// so walk a chunk faster than a workgroup with outputs; segment 0 is made
// shorter by the ratio below so that pass A ends about when its transitions
// do, and the other segments share the rest.  Measured on MI355X (d = 128)
// over ratios 0.4 .. 1.0: with mu, 0.7 at B1 H16 T16384 (268.6 -> 247.3 us)
// and 0.65-0.7 at B2 H16 T8192; without mu, 0.6 at both (207.6 -> 185.6 us
// at T16384).  ncs: chunks of segments 1 .. nseg - 2 (the last takes the
// rest, at most ncs); ncs0: chunks of segment 0.
constexpr double SEG0_RATIO_MOM = 0.7;
constexpr double SEG0_RATIO_NOMOM = 0.6;
void seg_lengths(int NC, int nseg, bool mom, int& ncs, int& ncs0)
{
    const double ratio = mom ? SEG0_RATIO_MOM : SEG0_RATIO_NOMOM;
    ncs = ncs0 = (NC + nseg - 1) / nseg;   // equal lengths, if no other fits
    for (int L = (int)(NC / (nseg - 1 + ratio)); L <= NC; ++L) {
        const int r = (int)(ratio * L + 0.5);
        const int L0 = r < 1 ? 1 : r > L ? L : r;
        const int rest = NC - L0 - (nseg - 2) * L;   // the last segment's chunks
        if (rest > L) continue;
        if (rest >= 1) {
            ncs = L;
            ncs0 = L0;
        }
        break;
    }
}
struct SegSizes {
    size_t ctab, states, trans;   // bytes, each a multiple of 256
};
SegSizes seg_sizes(int B, int T, int H, int Dk, int Dv, int nseg, bool mom)
{
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t nc = ((size_t)T + CH - 1) / CH;
    const size_t ncol = (size_t)Dv + (mom ? 2 : 1) * (size_t)Dk;
    SegSizes z;
    z.ctab = up((size_t)B * H * nc * ChunkTables::FLOATS * sizeof(float));
    z.states = up((size_t)B * nseg * H * Dk * Dv * sizeof(float));
    z.trans = up((size_t)B * (nseg - 2) * H * Dk * ncol * sizeof(float));
    return z;
}
}  // namespace

// Workspace of the segment scan: the coefficient tables, the segments' entry
// states (S and M) and their transitions (exit S and M).
size_t chunk_seg_workspace_bytes(int B, int T, int H, int Dk, int Dv, int nseg, bool mom)
{
    if (nseg < 3) return 0;
    const SegSizes z = seg_sizes(B, T, H, Dk, Dv, nseg, mom);
    return z.ctab + 2 * z.states + 2 * z.trans;
}

template <int DK, int DV>
static hipError_t launch_seg_t(const void* q, const void* k, const void* v, const float* alpha,
                               const float* mu, const float* eta, const float* beta,
                               const float* S0, const float* M0, void* O, float* ST, float* MT,
                               int B, int T, int H, int nseg, void* workspace, hipStream_t stream)
{
    const bool mom = mu != nullptr;
    const int NC = (T + CH - 1) / CH;
    const SegSizes z = seg_sizes(B, T, H, DK, DV, nseg, mom);
    char* w = static_cast<char*>(workspace);
    float* ctab = reinterpret_cast<float*>(w);
    SegArgs sg{};
    seg_lengths(NC, nseg, mom, sg.ncs, sg.ncs0);
    sg.nseg = nseg;
    sg.ncol = DV + (mom ? 2 : 1) * DK;
    sg.Sx = reinterpret_cast<float*>(w + z.ctab);
    sg.Mx = reinterpret_cast<float*>(w + z.ctab + z.states);
    sg.ES = reinterpret_cast<float*>(w + z.ctab + 2 * z.states);
    sg.EM = reinterpret_cast<float*>(w + z.ctab + 2 * z.states + z.trans);

    const unsigned nhg = (unsigned)((H + COEF_HEADS - 1) / COEF_HEADS);
    hipLaunchKernelGGL(chunk_coef_kernel, dim3((unsigned)B * nhg * (unsigned)NC),
                       dim3(COEF_HEADS * 64), 0, stream, alpha, mu, eta, beta, ctab, T, H, NC,
                       nhg);
    auto kern = mom ? chunk_fwd_seg_kernel<DK, DV, true> : chunk_fwd_seg_kernel<DK, DV, false>;
    const unsigned heads = (unsigned)B * (unsigned)H;
    constexpr unsigned NTILE = DV / 64;
    const unsigned ntall = NTILE + (mom ? 2u : 1u) * (DK / 64);   // transition tiles
    auto launch = [&](const SegArgs& a, unsigned ntr) {
        const unsigned nblk = a.nout + ntr;
        const int xcd_groups = nblk % 8 == 0 ? (int)(nblk / 8) : 0;
        hipLaunchKernelGGL(kern, dim3(nblk), dim3(2 * NT), 0, stream,
                           static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                           static_cast<const __bf16*>(v), ctab, S0, M0, static_cast<__bf16*>(O),
                           ST, MT, T, H, NC, xcd_groups, a);
    };
    // pass A: segment 0 with outputs, the transitions of 1 .. nseg - 2
    SegArgs a = sg;
    a.out_s0 = 0;
    a.out_ns = 1;
    a.nout = heads * NTILE;
    a.tr_s0 = 1;
    a.tr_ns = nseg - 2;
    launch(a, (unsigned)a.tr_ns * heads * ntall);
    // the entry states of segments 2 .. nseg - 1
    a.heads8 = heads % 8 == 0;
    auto comb = mom ? seg_combine_kernel<DK, DV, true> : seg_combine_kernel<DK, DV, false>;
    hipLaunchKernelGGL(comb, dim3(heads * (DV / 16)), dim3((mom ? 2 : 1) * DK * 4), 0, stream, a,
                       H);
    // pass B: segments 1 .. nseg - 1 with outputs
    SegArgs c = sg;
    c.out_s0 = 1;
    c.out_ns = nseg - 1;
    c.nout = (unsigned)(nseg - 1) * heads * NTILE;
    c.tr_s0 = 1;
    c.tr_ns = nseg - 2;
    launch(c, 0);
    return hipGetLastError();
}

// The bf16 forward as a segment scan of nseg >= 3 segments (chunk_seg_count).
// `workspace` holds chunk_seg_workspace_bytes(B, T, H, Dk, Dv, nseg, mu != NULL).
hipError_t launch_chunk_fused_seg(const void* q, const void* k, const void* v,
                                  const float* alpha, const float* mu, const float* eta,
                                  const float* beta, const float* S0, const float* M0, void* O,
                                  float* ST, float* MT, int B, int T, int H, int Dk, int Dv,
                                  int nseg, void* workspace, hipStream_t stream)
{
    if (Dk == 128 && Dv == 128)
        return launch_seg_t<128, 128>(q, k, v, alpha, mu, eta, beta, S0, M0, O, ST, MT, B, T, H,
                                      nseg, workspace, stream);
    if (Dk == 128 && Dv == 64)
        return launch_seg_t<128, 64>(q, k, v, alpha, mu, eta, beta, S0, M0, O, ST, MT, B, T, H,
                                     nseg, workspace, stream);
    if (Dk == 64 && Dv == 128)
        return launch_seg_t<64, 128>(q, k, v, alpha, mu, eta, beta, S0, M0, O, ST, MT, B, T, H,
                                     nseg, workspace, stream);
    return launch_seg_t<64, 64>(q, k, v, alpha, mu, eta, beta, S0, M0, O, ST, MT, B, T, H, nseg,
                                workspace, stream);
}

}  // namespace mdn
