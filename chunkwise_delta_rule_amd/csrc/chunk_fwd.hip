// chunk_fwd.hip -- chunkwise MDN forward on gfx950.
//
// The method ("MDN: Parallelizing Stepwise Momentum for Delta Linear
// Attention", slides Eqs. (7)-(9), (15)-(18), (40)-(42) with the Appendix C
// forms and the one-row-shifted residual mask of the backup frames; the
// reading notes on the same paper, Secs. 2.3-2.5), per chunk of C = 64 tokens
// with entry state (S0, M0), P = Diag(alpha) K and Khat = Diag(eta) K:
//
//   abar_i = prod_{r<=i} alpha_r        mubar_i = prod_{r<=i} mu_r
//   b_i    = alpha_i b_{i-1} + beta_i mubar_i  (= abar_i c_i)
//   gamma_{i,j} = sum_{r=j}^{i} beta_r (prod_{u=r+1}^{i} alpha_u)(prod_{u=j+1}^{r} mu_u)
//   L  = I + (P Khat^T) o Gamma^-       (Gamma^-: Gamma shifted down one row)
//   T  = L^{-1}
//   Vt = T [V - Diag(abar^-) P S0 + Diag(b^-) P M0]
//   O  = Diag(abar) Q S0 - Diag(b) Q M0 + [(Q Khat^T) o Gamma] Vt
//   S' = abar_C S0 - b_C M0 + [Diag(Gamma_C,:) Khat]^T Vt
//   M' = mubar_C M0 - [Diag(mubar_C / mubar) Khat]^T Vt
//
// with beta the gate of the memory update S_t = alpha_t S_{t-1} - beta_t M_t
// (beta = 1 when the caller gives none).  Gamma is formed by the
// division-free column recursion
//   gamma_{j,j} = beta_j,  m_{j,j} = 1,  m_{i,j} = mu_i m_{i-1,j},
//   gamma_{i,j} = alpha_i gamma_{i-1,j} + beta_i m_{i,j},
// which is the product-sum definition evaluated left to right; it needs no
// exp(-U_j) and no division by mubar, so mu = 0 is exact.  Note that
// Diag(abar^-) P = Diag(abar) K (alpha_i abar_{i-1} = abar_i).
//
// Two kernels:
//   chunk_prep_kernel  one workgroup per chunk, fully parallel.  Coefficients
//                      (one pass over the rows, gates broadcast across lanes),
//                      K K^T and Q K^T on MFMA, L, T = L^{-1} (16x16 diagonal
//                      blocks by forward substitution, off-diagonal blocks on
//                      fp32 MFMA), A = (Q Khat^T) o Gamma.  Writes T, A and the
//                      coefficient vectors to the workspace.
//   chunk_scan_kernel  one workgroup per (batch, head, 64 value columns),
//                      sequential over chunks.  Each wavefront keeps 16
//                      columns of S and M in fp32 MFMA accumulators for the
//                      whole sequence and feeds them, and its R and Vt, back
//                      into the next products directly from the accumulators.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "chunk_common.hpp"
#include "mfma.hpp"

namespace mdn {

template <typename E>
struct Workspace {
    E* T;
    E* A;
    float* vec;
};

template <typename E>
__host__ __device__ inline size_t ws_bytes(size_t nchunks)
{
    return nchunks * (2 * CH * CH * sizeof(E) + NVEC * CH * sizeof(float));
}

template <typename E>
__host__ __device__ inline Workspace<E> ws_carve(void* base, size_t nchunks)
{
    Workspace<E> w;
    char* p = static_cast<char*>(base);
    w.T = reinterpret_cast<E*>(p);
    p += nchunks * CH * CH * sizeof(E);
    w.A = reinterpret_cast<E*>(p);
    p += nchunks * CH * CH * sizeof(E);
    w.vec = reinterpret_cast<float*>(p);
    return w;
}

// Column swizzle of the transposed K copy K^T[d][c]: groups of 4 chunk rows c
// are XOR-permuted by the row d, so that the transposing writes (8 values of
// one chunk row per thread) spread over the LDS banks instead of landing 16
// deep on one bank, while every aligned group of 4 stays contiguous for the
// 8-byte fragment reads.
__device__ __forceinline__ int kt_swz(int d, int c) { return c ^ (4 * ((d >> 3) & 7)); }

// Prefetch of CH rows x D columns of a row-major [*, row_stride] array into
// registers (16-byte vectors; rows >= n read as zero), stored later into an
// LDS array with row stride LD.
template <typename E, int D>
struct RowTile {
    static constexpr int EPV = 16 / sizeof(E);   // elements per vector
    static constexpr int VPR = D / EPV;          // vectors per row
    static constexpr int NV = CH * VPR / NT;     // vectors per thread
    static_assert(CH * VPR % NT == 0, "tile must split evenly over the workgroup");
    uint4 r[NV];
    int n = CH;

    // base: row 0 of the tile (wave-uniform).  Rows >= n read row n - 1 (so
    // every load is in bounds and none is predicated) and are zeroed when
    // stored, so the loads can stay in flight until then.
    __device__ __forceinline__ void load(const E* __restrict__ base, unsigned row_stride, int rows,
                                         int tid)
    {
        n = rows;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int idx = tid + NT * u;
            const int row = idx / VPR;
            const unsigned col = (unsigned)(idx % VPR) * EPV;
            const unsigned off = (unsigned)min(row, n - 1) * row_stride + col;
            r[u] = *reinterpret_cast<const uint4*>(base + off);
        }
    }
    __device__ __forceinline__ uint4 get(int u, int tid) const
    {
        // bitwise mask rather than a select, so no branch is generated
        const unsigned m = (tid + NT * u) / VPR < n ? ~0u : 0u;
        return uint4{r[u].x & m, r[u].y & m, r[u].z & m, r[u].w & m};
    }
    template <int LD>
    __device__ __forceinline__ void store(E* dst, int tid) const
    {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int idx = tid + NT * u;
            *reinterpret_cast<uint4*>(dst + (idx / VPR) * LD + (idx % VPR) * EPV) = get(u, tid);
        }
    }
    // transposed store: element (row, col) goes to dst[col * LD + kt_swz(col, row)]
    template <int LD>
    __device__ __forceinline__ void store_transposed(E* dst, int tid) const
    {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int idx = tid + NT * u;
            const int row = idx / VPR;
            const int col = (idx % VPR) * EPV;
            const uint4 x = get(u, tid);
            const E* e = reinterpret_cast<const E*>(&x);
#pragma unroll
            for (int j = 0; j < EPV; ++j) dst[(col + j) * LD + kt_swz(col + j, row)] = e[j];
        }
    }
};

__device__ __forceinline__ float lane_bcast(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// ---------------------------------------------------------------------------
// Per-chunk preparation
// ---------------------------------------------------------------------------
// With bf16 I/O, Q never enters LDS (each wavefront loads its own row tile's
// MFMA fragments from memory) and L is written over Gamma once the masks have
// read it: region0 holds K, later T; region1 Gamma, later L.  That is 35.9 KB
// at DK = 128, four workgroups per CU.  With fp32 I/O, region0 holds K and Q,
// later L and T.
template <typename E, int DK>
struct PrepSmem {
    static constexpr bool QREG = sizeof(E) == 2;
    static constexpr int LDK = DK + Mma<E>::PAD;
    static constexpr int LDG = CH + 4;   // fp32 C x C matrices; 4 rows apart = 16 banks apart
    static constexpr size_t kq_bytes = (QREG ? 1 : 2) * CH * LDK * sizeof(E);
    static constexpr size_t lt_bytes = (QREG ? 1 : 2) * CH * LDG * sizeof(float);
    static constexpr size_t region0 = kq_bytes > lt_bytes ? kq_bytes : lt_bytes;
    static constexpr size_t region1 = CH * LDG * sizeof(float);
};

template <typename E, int DK>
__global__ __launch_bounds__(NT) void chunk_prep_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const float* __restrict__ alpha,
    const float* __restrict__ mu, const float* __restrict__ eta, const float* __restrict__ beta,
    E* __restrict__ Tw, E* __restrict__ Aw, float* __restrict__ Vw, int T, int H, int NC)
{
    using MM = Mma<E>;
    using MF = Mma<float>;
    using SM = PrepSmem<E, DK>;
    constexpr int LDK = SM::LDK;
    constexpr int LDG = SM::LDG;
    constexpr bool QREG = SM::QREG;

    __shared__ __align__(16) char smem0[SM::region0];
    __shared__ __align__(16) char smem1[SM::region1];
    __shared__ __align__(16) float al[CH];
    __shared__ __align__(16) float mus[CH];
    __shared__ __align__(16) float et[CH];
    __shared__ __align__(16) float bts[CH];
    E* Ks = reinterpret_cast<E*>(smem0);
    E* Qs = Ks + CH * LDK;   // fp32 I/O only
    float* Gam = reinterpret_cast<float*>(smem1);
    float* Ls = QREG ? Gam : reinterpret_cast<float*>(smem0);
    float* Ts = QREG ? reinterpret_cast<float*>(smem0) : Ls + CH * LDG;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;

    const size_t ch = blockIdx.x;                 // (b * H + h) * NC + c
    const int c = (int)(ch % NC);
    const int h = (int)((ch / NC) % H);
    const int b = (int)(ch / ((size_t)NC * H));
    const int t0 = c * CH;
    const int n = min(CH, T - t0);
    const size_t tok0 = ((size_t)b * T + t0) * H + h;   // (b, t0, h)

    // gates of this chunk, one row per lane (rows >= n: alpha 1, mu 0, eta 0,
    // beta 0); beta is 1 when no beta gate is given.  K and Q are loaded next
    // into registers (bf16: Q as this wavefront's MFMA fragments, never
    // stored) and K (fp32: K and Q) reaches LDS only after the coefficient
    // pass, which needs the gates alone, so their latency overlaps it.
    float a_l = 1.f, m_l = 0.f, e_l = 0.f, s_l = 0.f;
    if (lane < n) {
        const size_t g = tok0 + (size_t)lane * H;
        a_l = alpha[g];
        m_l = mu ? mu[g] : 0.f;   // NULL: mu = 0
        e_l = eta[g];
        s_l = beta ? beta[g] : 1.f;
    }
    RowTile<E, DK> kt, qt;
    kt.load(k + tok0 * DK, (unsigned)(H * DK), n, tid);
    // bf16: this lane's A fragments of Q K^T, row 16 wave + l16 (rows >= n
    // read row n - 1 and are zeroed where used)
    typename MM::frag aQf[DK / MM::KSTEP];
    const int qrow = 16 * wave + l16;
    if constexpr (QREG) {
        const E* qr = q + tok0 * DK + (size_t)min(qrow, n - 1) * (H * DK) + MM::KW * lg;
#pragma unroll
        for (int s = 0; s < DK / MM::KSTEP; ++s) aQf[s] = MM::load(qr + MM::KSTEP * s);
    } else {
        qt.load(q + tok0 * DK, (unsigned)(H * DK), n, tid);
    }
    if (wave == 0) {
        al[lane] = a_l;
        mus[lane] = m_l;
        et[lane] = e_l;
        bts[lane] = s_l;
    }
    __syncthreads();

    // ---- coefficients, Gamma by 16-row blocks: block w (rows r0 = 16 w ..
    //      r0 + 15) on wavefront w, lane j carrying the Gamma column j.  For
    //      r > j the column runs m_{r,j} = mu_r m_{r-1,j},
    //      gamma_{r,j} = alpha_r gamma_{r-1,j} + beta_r m_{r,j} (gamma_jj = beta_j,
    //      m_jj = 1).  Inside a block this is linear in the entry state
    //      (gamma, m) at row r0 - 1, with the same coefficients for every
    //      column j < r0: gamma_{r,j} = a_r gamma_in + b_r m_in, m_{r,j} = c_r m_in,
    //      where c_r = prod_{u=r0..r} mu_u, a_r = prod alpha_u and
    //      b_r = alpha_r b_{r-1} + beta_r c_r.  Phase 1: every wavefront forms its
    //      (a_r, b_r, c_r) and the columns that start inside its block; phase
    //      2: it carries the earlier columns' exit states through the blocks
    //      between.  abar_i = prod_{u<=i} alpha_u is the product of the earlier
    //      blocks' a and the lane's own a_i.  Since
    //      mubar_r = mu_0 prod_{u=1..r} mu_u, column 0 gives b_i = mu_0 gamma_{i,0}
    //      and mubar_{n-1} = mu_0 m_{n-1,0}.  Rows >= n carry neutral gates
    //      and are written as zero.
    //      Gamma's row padding (columns 64..67) holds per-column values
    //      exchanged between the phases: a block's exit state (gamma, m) of
    //      its own columns, abar and m_{n-1,j}.
    float* Vch = Vw + ch * NVEC * CH;
    __shared__ float comp[4][4];                 // a, b, c of each block's last row
    constexpr int XG = 64, XM = 65, XAB = 66, XMF = 67;
    const int r0 = 16 * wave;
    float pa[16], pb[16], pc[16], mloc[16];
    float abr = 1.f;
    {
        float ga[16], gm[16], gs[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float4 a4 = *reinterpret_cast<const float4*>(al + r0 + 4 * u);
            const float4 m4 = *reinterpret_cast<const float4*>(mus + r0 + 4 * u);
            const float4 s4 = *reinterpret_cast<const float4*>(bts + r0 + 4 * u);
            ga[4 * u + 0] = a4.x; ga[4 * u + 1] = a4.y; ga[4 * u + 2] = a4.z; ga[4 * u + 3] = a4.w;
            gm[4 * u + 0] = m4.x; gm[4 * u + 1] = m4.y; gm[4 * u + 2] = m4.z; gm[4 * u + 3] = m4.w;
            gs[4 * u + 0] = s4.x; gs[4 * u + 1] = s4.y; gs[4 * u + 2] = s4.z; gs[4 * u + 3] = s4.w;
        }
        float ca = 1.f, cb = 0.f, cc = 1.f;      // the block's coefficients
        float gl = 0.f, ml = 1.f;                // column `lane` if it starts in this block
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int r = r0 + u;
            cc *= gm[u];
            ca *= ga[u];
            cb = ga[u] * cb + gs[u] * cc;
            pa[u] = ca;
            pb[u] = cb;
            pc[u] = cc;
            abr = r == lane ? ca : abr;
            const bool below = r > lane;
            const float ml_n = below ? ml * gm[u] : 1.f;
            const float gl_n = below ? ga[u] * gl + gs[u] * ml_n : (r == lane ? gs[u] : 0.f);
            ml = ml_n;
            gl = gl_n;
            mloc[u] = ml_n;
            // columns j >= r0 are final here (zero above the diagonal)
            if (lane >= r0) Gam[r * LDG + lane] = r < n ? gl_n : 0.f;
        }
        if (lane >= r0 && lane < r0 + 16) {
            Gam[lane * LDG + XG] = gl;
            Gam[lane * LDG + XM] = ml;
        }
        if (lane == 0) {
            comp[wave][0] = ca;
            comp[wave][1] = cb;
            comp[wave][2] = cc;
        }
    }
    __syncthreads();
    {
        // phase 2: columns j < r0 from the exit state of their own block,
        // carried through the blocks between
        float gi = 0.f, mi = 0.f;
        if (lane < r0) {
            const int kb = lane >> 4;
            gi = Gam[lane * LDG + XG];
            mi = Gam[lane * LDG + XM];
#pragma unroll
            for (int kx = 1; kx < 3; ++kx) {
                if (kx > kb && kx < wave) {
                    const float g2 = comp[kx][0] * gi + comp[kx][1] * mi;
                    mi = comp[kx][2] * mi;
                    gi = g2;
                }
            }
#pragma unroll
            for (int u = 0; u < 16; ++u)
                Gam[(r0 + u) * LDG + lane] = r0 + u < n ? pa[u] * gi + pb[u] * mi : 0.f;
        }
        // abar of the rows of this block
        float pre = 1.f;
#pragma unroll
        for (int kx = 0; kx < 3; ++kx)
            if (kx < wave) pre *= comp[kx][0];
        if (lane >= r0 && lane < r0 + 16) Gam[lane * LDG + XAB] = pre * abr;
        // m_{n-1,j} from the block that holds row n - 1
        if (wave == (n - 1) >> 4) {
            const int un = (n - 1) & 15;
            float pcu = 0.f, mlu = 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                pcu = u == un ? pc[u] : pcu;
                mlu = u == un ? mloc[u] : mlu;
            }
            Gam[lane * LDG + XMF] = lane < r0 ? pcu * mi : mlu;
        }
    }

    kt.template store<LDK>(Ks, tid);
    if constexpr (!QREG) qt.template store<LDK>(Qs, tid);
    __syncthreads();

    // ---- G = K K^T and P = Q K^T on the lower block triangle: wave w owns
    //      row tile w.  The accumulators hold the transposed tiles: lane
    //      (l16, lg) ends with row i = 16 w + l16, columns 16 ct + 4 lg .. + 3,
    //      so every later access of a row is one 16-byte piece.
    f32x4 accG[4], accP[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) accG[ct] = accP[ct] = zero4();
#pragma unroll
    for (int ks = 0; ks < DK; ks += MM::KSTEP) {
        const int kk = ks + MM::KW * lg;
        const auto aK = MM::load(Ks + (16 * wave + l16) * LDK + kk);
        typename MM::frag aQ;
        if constexpr (QREG)
            aQ = qrow < n ? aQf[ks / MM::KSTEP] : typename MM::frag{};
        else
            aQ = MM::load(Qs + (16 * wave + l16) * LDK + kk);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            if (ct <= wave) {
                const auto bK = MM::load(Ks + (16 * ct + l16) * LDK + kk);
                accG[ct] = MM::mma(bK, aK, accG[ct]);
                accP[ct] = MM::mma(bK, aQ, accP[ct]);
            }
        }
    }
    __syncthreads();   // Gamma ready; K and Q no longer read

    if (wave == 0) {
        const float mu0 = mus[0];
        const bool live = lane < n;
        const float bi = live ? mu0 * Gam[lane * LDG] : 0.f;
        const float bprev = live && lane >= 1 ? mu0 * Gam[(lane - 1) * LDG] : 0.f;
        const float ab = Gam[lane * LDG + XAB];
        const float g = Gam[(n - 1) * LDG + lane];     // gamma_{n-1, lane}
        const float mj = Gam[lane * LDG + XMF];        // m_{n-1, lane}
        Vch[V_ABAR * CH + lane] = live ? ab : 0.f;
        Vch[V_AB1 * CH + lane] = live ? a_l * bprev : 0.f;
        Vch[V_B * CH + lane] = bi;
        Vch[V_WS * CH + lane] = live ? e_l * g : 0.f;
        Vch[V_WM * CH + lane] = live ? e_l * mj : 0.f;
        // [abar_{n-1}, b_{n-1}, mubar_{n-1}] from lanes n-1 and 0
        const float ab_last = lane_bcast(ab, n - 1);
        const float mj0 = lane_bcast(mj, 0);
        const float b_last = lane_bcast(bi, n - 1);
        float scal = 0.f;
        if (lane == 0) scal = ab_last;
        if (lane == 1) scal = b_last;
        if (lane == 2) scal = mu0 * mj0;
        Vch[V_SCAL * CH + lane] = scal;
    }

    // ---- L = I + (P Khat^T) o Gamma^- into LDS (bf16: over Gamma, after
    //      every wavefront has read it; fp32: over K/Q, no longer read) and
    //      A = (Q Khat^T) o Gamma straight to the workspace, 4 columns of row
    //      i per lane
    E* Ach = Aw + ch * CH * CH;
    {
        f32x4 lrow[4];
        const int i = 16 * wave + l16;
        const float ai = al[i];
        const float* g0row = Gam + i * LDG;
        const float* gmrow = Gam + max(i - 1, 0) * LDG;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int j0 = 16 * ct + 4 * lg;
            f32x4 lv = zero4(), av = zero4();
            if (ct <= wave) {   // wave-uniform; the per-lane masks are selects
                const f32x4 g0 = *reinterpret_cast<const f32x4*>(g0row + j0);
                const f32x4 gm1 = *reinterpret_cast<const f32x4*>(gmrow + j0);
                const f32x4 e4 = *reinterpret_cast<const f32x4*>(et + j0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = j0 + r;
                    lv[r] = j < i ? ai * accG[ct][r] * e4[r] * gm1[r] : (i == j ? 1.f : 0.f);
                    av[r] = j <= i ? accP[ct][r] * e4[r] * g0[r] : 0.f;
                }
            }
            lrow[ct] = lv;
            if constexpr (!QREG) *reinterpret_cast<f32x4*>(Ls + i * LDG + j0) = lv;
            store4<E>(Ach + i * CH + j0, av[0], av[1], av[2], av[3]);
        }
        if constexpr (QREG) {
            __syncthreads();   // Gamma no longer read
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                *reinterpret_cast<f32x4*>(Ls + i * LDG + 16 * ct + 4 * lg) = lrow[ct];
        }
    }
    __syncthreads();

    // ---- T = L^{-1}.  Diagonal 16x16 blocks by column-oriented forward
    //      substitution (wave w, lanes 0..15 = columns of block w): once t_j
    //      is final, every later row subtracts its multiple, so the updates
    //      of one step are independent ...
    if (lane < 16) {
        const int base = 16 * wave;
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = (i == lane) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 15; ++j) {
#pragma unroll
            for (int i = j + 1; i < 16; ++i) t[i] -= Ls[(base + i) * LDG + base + j] * t[j];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Ts[(base + i) * LDG + base + lane] = t[i];
    }
    __syncthreads();
    // ... then the blocks below the diagonal, by halves: with
    //      L = [[L1, 0], [L21, L2]] (32 x 32 blocks) and T1 = L1^-1, T2 = L2^-1,
    //      T = [[T1, 0], [-T2 L21 T1, T2]], and the same once more inside T1 and
    //      T2 (T_10 = -D_1 L_10 D_0, T_32 = -D_3 L_32 D_2).  Three dependent
    //      steps of 16 x 16 products on fp32 MFMA, spread over the wavefronts:
    //      (1) T_10 and T_32; (2) Y = L21 T1, one block per wavefront, kept in
    //      L's upper right 32 x 32 (zero, never read); (3) -T2 Y, one block per
    //      wavefront.  Only blocks on or below the diagonal of T are read.
    //      acc += A_blk(I, KA) B_blk(KB, J) for row-major A, B in LDS (16 x 16
    //      blocks; A's block column KA against B's block row KB):
    auto blk_mma = [&](const float* Am, int I, int KA, const float* Bm, int KB, int J,
                       f32x4 acc) {
        f32x4 a1 = zero4();
#pragma unroll
        for (int kk = 0; kk < 16; kk += 2 * MF::KSTEP) {
            acc = MF::mma(Am[(16 * I + l16) * LDG + 16 * KA + kk + lg],
                          Bm[(16 * KB + kk + lg) * LDG + 16 * J + l16], acc);
            a1 = MF::mma(Am[(16 * I + l16) * LDG + 16 * KA + kk + 4 + lg],
                         Bm[(16 * KB + kk + 4 + lg) * LDG + 16 * J + l16], a1);
        }
        return acc + a1;
    };
    // -D_I X with X in accumulators (the B operand in k-permuted order:
    // step s covers k = 4 lg + s, this lane's element s)
    auto neg_diag_times = [&](int I, const f32x4& x) {
        f32x4 t = zero4();
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
            t = MF::mma(Ts[(16 * I + l16) * LDG + 16 * I + 4 * lg + s2], -x[s2], t);
        return t;
    };
    auto store_blk = [&](float* M, int I, int J, const f32x4& t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) M[(16 * I + 4 * lg + r) * LDG + 16 * J + l16] = t[r];
    };
    if (wave < 2) {
        const int I = 1 + 2 * wave, J = 2 * wave;              // (1, 0) or (3, 2)
        store_blk(Ts, I, J, neg_diag_times(I, blk_mma(Ls, I, J, Ts, J, J, zero4())));
    }
    __syncthreads();
    float* const Ys = Ls + 32;                                 // Y_{I-2, J} at rows 16 (I-2), columns 32 + 16 J
    {
        const int I = 2 + (wave >> 1), J = wave & 1;
        f32x4 y = blk_mma(Ls, I, 1, Ts, 1, J, zero4());        // L_{I,1} T1_{1,J}
        if (J == 0) y = blk_mma(Ls, I, 0, Ts, 0, 0, y);        // + L_{I,0} D_0
        store_blk(Ys, I - 2, J, y);
    }
    __syncthreads();
    {
        const int I = 2 + (wave >> 1), J = wave & 1;
        f32x4 t = blk_mma(Ts, I, 2, Ys, 0, J, zero4());         // T2_{I,2} Y_{2,J}: D_2 or T_32
        if (I == 3) t = blk_mma(Ts, 3, 3, Ys, 1, J, t);         // + D_3 Y_{3,J}
        store_blk(Ts, I, J, -t);
    }
    __syncthreads();

    // ---- write T (zero above the block diagonal) in the I/O type
    E* Tch = Tw + ch * CH * CH;
    constexpr int EPV = 16 / sizeof(E);
    for (int idx = tid; idx < CH * CH / EPV; idx += NT) {
        const int row = (idx * EPV) / CH;
        const int col = (idx * EPV) % CH;
        const bool upper = (col >> 4) > (row >> 4);
        alignas(16) E tv[EPV];
#pragma unroll
        for (int j = 0; j < EPV; ++j) {
            const float x = Ts[row * LDG + col + j];   // stale above the diagonal: masked
            tv[j] = to_elem<E>(upper ? 0.f : x);
        }
        *reinterpret_cast<uint4*>(Tch + row * CH + col) = *reinterpret_cast<const uint4*>(tv);
    }
}

// ---------------------------------------------------------------------------
// Sequential scan over chunks.  One workgroup per (batch, head, 64 value
// columns); wavefront w owns 16 of those columns of S and M for the whole
// sequence.  Everything a wavefront computes for its columns (K S, Q S, R,
// Vt, O, the new S and M) depends only on its own columns and on the
// chunk's shared operands (K, Q, V, T, A, coefficients) in LDS, so the four
// wavefronts never wait for each other inside a chunk: they synchronise only
// around the staging of the next chunk, whose global loads are issued before
// the current chunk's arithmetic (bf16) so their latency is hidden.
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
struct ScanSmem {
    static constexpr int TV = 64;
    static constexpr int LDK = DK + Mma<E>::PAD;
    static constexpr int LDV = TV + Mma<E>::PAD;
    static constexpr int LDC = CH + Mma<E>::PAD;
    static constexpr bool KT_COPY = sizeof(E) == 2;
};

template <typename E, int DK, int DV>
__global__ __launch_bounds__(NT) void chunk_scan_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ Tw, const E* __restrict__ Aw, const float* __restrict__ Vw,
    const float* S0, const float* M0, E* __restrict__ O, E* __restrict__ Vto, float* ST,
    float* MT, int T, int H, int NC, int xcd_groups)
{
    using MM = Mma<E>;
    using SM = ScanSmem<E, DK, DV>;
    constexpr int TV = SM::TV;
    constexpr int NTILE = DV / TV;
    constexpr int LDK = SM::LDK;
    constexpr int LDV = SM::LDV;
    constexpr int LDC = SM::LDC;
    constexpr bool KT_COPY = SM::KT_COPY;
    constexpr bool PREFETCH = sizeof(E) == 2;
    constexpr int RT = DK / 16;            // row tiles of the state
    constexpr int SK = DK / MM::PERM_K;    // k-steps over d
    constexpr int SC = CH / MM::PERM_K;    // k-steps over the chunk rows
    static_assert(DV % TV == 0, "value tile");

    __shared__ __align__(16) E Ks[CH * LDK];
    __shared__ __align__(16) E Qs[CH * LDK];
    __shared__ __align__(16) E KTs[KT_COPY ? DK * LDC : 8];
    __shared__ __align__(16) E Vs[CH * LDV];
    __shared__ __align__(16) E Ts[CH * LDC];
    __shared__ __align__(16) E As[CH * LDC];
    __shared__ __align__(16) float vecs[6 * CH];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;

    // Workgroups are dispatched round-robin over the 8 XCDs.  When the grid
    // is a multiple of 8, renumber so that consecutive logical ids (the value
    // tiles of one head, which read the same K, Q, T and A) run on one XCD
    // and share its L2.
    unsigned bid = blockIdx.x;
    if (xcd_groups > 0) bid = (bid % 8u) * (unsigned)xcd_groups + bid / 8u;
    const int tile = (int)(bid % NTILE);
    const int bh = (int)(bid / NTILE);     // b * H + h
    const int h = bh % H;
    const int b = bh / H;
    const int wcol = tile * TV + 16 * wave;   // first value column of this wavefront

    // the state columns of this wavefront: rows 16 rt + 4 lg + r, column wcol + l16
    f32x4 Sa[RT], Ma[RT];
    const size_t sbase = (size_t)bh * DK * DV;
    auto load_state = [&](f32x4* X, const float* src) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                X[rt][r] = src ? src[sbase + (size_t)(16 * rt + 4 * lg + r) * DV + wcol + l16] : 0.f;
        }
    };
    if (S0) load_state(Sa, S0); else load_state(Sa, nullptr);
    if (M0) load_state(Ma, M0); else load_state(Ma, nullptr);

    RowTile<E, DK> pk, pq;
    RowTile<E, TV> pv;
    RowTile<E, CH> pt, pa;
    float4 pvec = {0.f, 0.f, 0.f, 0.f};
    auto fetch = [&](int c) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const size_t tok0 = ((size_t)b * T + t0) * H + h;
        const size_t chn = (size_t)bh * NC + c;
        pk.load(k + tok0 * DK, (unsigned)(H * DK), n, tid);
        pq.load(q + tok0 * DK, (unsigned)(H * DK), n, tid);
        pv.load(v + tok0 * DV + tile * TV, (unsigned)(H * DV), n, tid);
        pt.load(Tw + chn * CH * CH, CH, CH, tid);
        pa.load(Aw + chn * CH * CH, CH, CH, tid);
        if (tid < 6 * CH / 4) pvec = reinterpret_cast<const float4*>(Vw + chn * NVEC * CH)[tid];
    };
    if (PREFETCH) fetch(0);

    for (int c = 0; c < NC; ++c) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const size_t tok0 = ((size_t)b * T + t0) * H + h;

        if (!PREFETCH) fetch(c);
        __syncthreads();   // the previous chunk's LDS operands are no longer read
        pk.template store<LDK>(Ks, tid);
        if (KT_COPY) pk.template store_transposed<LDC>(KTs, tid);
        pq.template store<LDK>(Qs, tid);
        pv.template store<LDV>(Vs, tid);
        pt.template store<LDC>(Ts, tid);
        pa.template store<LDC>(As, tid);
        if (tid < 6 * CH / 4) reinterpret_cast<float4*>(vecs)[tid] = pvec;
        __syncthreads();
        if (PREFETCH && c + 1 < NC) fetch(c + 1);

        // (1) X = K [S | M], Y = Q [S | M] for all chunk rows, this
        //     wavefront's 16 columns; the state is the B operand straight
        //     from its accumulators
        f32x4 xs[4], xm[4], ys[4], ym[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) xs[ct] = xm[ct] = ys[ct] = ym[ct] = zero4();
#pragma unroll
        for (int s = 0; s < SK; ++s) {
            const auto bS = MM::from_acc(Sa, s);
            const auto bM = MM::from_acc(Ma, s);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const auto aK = MM::load_perm(Ks + (16 * ct + l16) * LDK, s, lg);
                const auto aQ = MM::load_perm(Qs + (16 * ct + l16) * LDK, s, lg);
                xs[ct] = MM::mma(aK, bS, xs[ct]);
                xm[ct] = MM::mma(aK, bM, xm[ct]);
                ys[ct] = MM::mma(aQ, bS, ys[ct]);
                ym[ct] = MM::mma(aQ, bM, ym[ct]);
            }
        }

        // (2) R = V - Diag(abar) K S0 + Diag(alpha b^-) K M0 and the entry-state
        //     part of O, element (row 16 ct + 4 lg + r, column l16)
        f32x4 R[4], Oa[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ct + 4 * lg + r;
                const float ab = vecs[V_ABAR * CH + i];
                R[ct][r] = to_f32(Vs[i * LDV + 16 * wave + l16]) - ab * xs[ct][r] +
                           vecs[V_AB1 * CH + i] * xm[ct][r];
                Oa[ct][r] = ab * ys[ct][r] - vecs[V_B * CH + i] * ym[ct][r];
            }
        }

        // (3) Vt = T R
        f32x4 Vt[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) Vt[it] = zero4();
#pragma unroll
        for (int s = 0; s < SC; ++s) {
            const auto bR = MM::from_acc(R, s);
#pragma unroll
            for (int it = 0; it < 4; ++it)
                Vt[it] = MM::mma(MM::load_perm(Ts + (16 * it + l16) * LDC, s, lg), bR, Vt[it]);
        }

        // the residuals of every token, when asked for (Vto: [B, T, H, DV] like O)
        if (Vto) {
            E* Vb = Vto + tok0 * DV + wcol + l16;
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * it + 4 * lg + r;
                    if (i < n) Vb[(size_t)i * H * DV] = to_elem<E>(Vt[it][r]);
                }
        }

        // (4) O = entry-state part + A Vt; rows < n to HBM
#pragma unroll
        for (int s = 0; s < SC; ++s) {
            const auto bV = MM::from_acc(Vt, s);
#pragma unroll
            for (int it = 0; it < 4; ++it)
                Oa[it] = MM::mma(MM::load_perm(As + (16 * it + l16) * LDC, s, lg), bV, Oa[it]);
        }
        {
            E* Ob = O + tok0 * DV + wcol + l16;
            const unsigned ostride = (unsigned)(H * DV);
            if (n == CH) {
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Ob[(unsigned)(16 * it + 4 * lg + r) * ostride] = to_elem<E>(Oa[it][r]);
            } else {
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = 16 * it + 4 * lg + r;
                        if (i < n) Ob[(unsigned)i * ostride] = to_elem<E>(Oa[it][r]);
                    }
            }
        }

        // (5) carried state from the old S0, M0:
        //     S' = abar_n S0 - b_n M0 + K^T Diag(eta gamma_n) Vt
        //     M' = mubar_n M0 - K^T Diag(eta mubar_n / mubar) Vt
        const float abn = vecs[V_SCAL * CH + 0];
        const float bn = vecs[V_SCAL * CH + 1];
        const float mbn = vecs[V_SCAL * CH + 2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            Sa[rt] = abn * Sa[rt] - bn * Ma[rt];
            Ma[rt] = mbn * Ma[rt];
        }
#pragma unroll
        for (int s = 0; s < SC; ++s) {
            const auto bS = MM::from_acc_scaled(Vt, s, lg, vecs + V_WS * CH, 1.f);
            const auto bM = MM::from_acc_scaled(Vt, s, lg, vecs + V_WM * CH, -1.f);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                typename MM::frag aK;
                if constexpr (KT_COPY) {
                    // row d = 16 rt + l16; its chunk-row groups are XOR-swizzled
                    const int d = 16 * rt + l16;
                    aK = MM::load_perm_xor(KTs + d * LDC, s, lg, 4 * ((d >> 3) & 7));
                } else {
                    aK = Ks[MM::perm_row(s, lg, 0) * LDK + 16 * rt + l16];
                }
                Sa[rt] = MM::mma(aK, bS, Sa[rt]);
                Ma[rt] = MM::mma(aK, bM, Ma[rt]);
            }
        }
    }

    auto store_state = [&](float* dst, const f32x4* X) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[sbase + (size_t)(16 * rt + 4 * lg + r) * DV + wcol + l16] = X[rt][r];
        }
    };
    if (ST) store_state(ST, Sa);
    if (MT) store_state(MT, Ma);
}


// ---------------------------------------------------------------------------
// bf16 scan.  Same mathematics and column ownership as chunk_scan_kernel;
// one wavefront per SIMD is all the head-tile parallelism a layer has, so
// the compute wavefronts are kept free of everything but their own chain.
//
//  * Roles.  Eight wavefronts: 0..3 compute (wavefront w owns 16 of the 64
//    value columns of S and M for the whole sequence), 4..7 stage.  While
//    the compute wavefronts work on chunk c, the staging wavefronts bring
//    chunk c + 1 into the other LDS buffer with direct global-to-LDS loads
//    only (K, Q, V, T, A and the coefficient vectors, row-major); the
//    compute wavefronts read K^T and V in the layouts they need with
//    transposing LDS reads.  One barrier per chunk hands the buffers over.
//  * Row order.  The accumulator slot (tile t, lane group g, element j) of
//    the state (rows d) and of the chunk-row results (rows c) stands for
//    physical row phys_row(16 t + 4 g + j): inside each block of 32 rows,
//    slots 4g + j and 16 + 4g + j hold rows 8g + j and 8g + 4 + j.  A k-step
//    fed from accumulator tiles 2s and 2s + 1 then covers physical rows
//    32s + 8g + (0..7), so every A fragment is 8 contiguous elements of one
//    row: one 16-byte LDS read.
//  * Outputs are produced transposed, O^T = S^T Q^T + Vt^T A^T, so that a
//    lane ends with 4 adjacent columns of one output row: one 8-byte store.
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct ScanBf16Layout {
    using LK = TileLayout<DK * 2>;          // K, Q rows
    using LC = TileLayout<CH * 2>;          // T, A rows and K^T rows
    static constexpr int TV = 64;           // value columns per workgroup
    static constexpr int OFF_Q = LK::BYTES;
    static constexpr int OFF_T = 2 * LK::BYTES;
    static constexpr int OFF_A = OFF_T + LC::BYTES;
    static constexpr int OFF_V = OFF_A + LC::BYTES;   // 64 rows x 64 value columns
    static constexpr int OFF_VEC = OFF_V + LC::BYTES;
    static constexpr int BUF_BYTES = OFF_VEC + 6 * CH * 4;
    // byte distance between the rows 32 s + x and x of a K tile
    static constexpr int KSTEP_ROWS = 32 * (DK * 2) + (32 / LK::G) * LK::PAD;
};

template <int DK, int DV>
__global__ __launch_bounds__(2 * NT) void chunk_scan_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ Tw, const __bf16* __restrict__ Aw, const float* __restrict__ Vw,
    const float* S0, const float* M0, __bf16* __restrict__ O, float* ST, float* MT, int T,
    int H, int NC, int xcd_groups)
{
    using E = __bf16;
    using MM = Mma<E>;
    using L = ScanBf16Layout<DK, DV>;
    using LK = typename L::LK;
    using LC = typename L::LC;
    constexpr int TV = L::TV;
    constexpr int NTILE = DV / TV;
    constexpr int RT = DK / 16;             // state row tiles
    constexpr int SK = DK / 32;             // k-steps over d
    constexpr int SC = CH / 32;             // k-steps over the chunk rows
    static_assert(DV % TV == 0, "value tile");

    __shared__ __align__(16) char buf[2][L::BUF_BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;

    unsigned bid = blockIdx.x;
    if (xcd_groups > 0) bid = (bid % 8u) * (unsigned)xcd_groups + bid / 8u;
    const int tile = (int)(bid % NTILE);
    const int bh = (int)(bid / NTILE);
    const int h = bh % H;
    const int b = bh / H;

    if (wave >= 4) {
        // ---------------- staging wavefronts ----------------
        const int hw = wave - 4;
        const unsigned kq_stride = (unsigned)(H * DK);
        const unsigned kq_lane = LK::lane_offset(kq_stride, lane);
        const unsigned c_lane = LC::lane_offset(CH, lane);
        const unsigned v_stride = (unsigned)(H * DV);
        const unsigned v_lane = LC::lane_offset(v_stride, lane);
        auto stage = [&](int c, int bi) {
            const int n = min(CH, T - c * CH);
            const size_t tok0 = ((size_t)b * T + c * CH) * H + h;
            const size_t chn = (size_t)bh * NC + c;
            char* B = buf[bi];
            LK::load(B, k + tok0 * DK, kq_stride, kq_lane, n, hw, lane);
            LK::load(B + L::OFF_Q, q + tok0 * DK, kq_stride, kq_lane, n, hw, lane);
            LC::load(B + L::OFF_T, Tw + chn * CH * CH, CH, c_lane, CH, hw, lane);
            LC::load(B + L::OFF_A, Aw + chn * CH * CH, CH, c_lane, CH, hw, lane);
            // this tile's 64 value columns of V (rows >= n read row n - 1)
            LC::load(B + L::OFF_V, v + tok0 * DV + tile * TV, v_stride, v_lane, n, hw, lane);
            // coefficient vectors: 6 x 64 floats = 96 pieces of 16 bytes
            if (hw == 0 || (hw == 1 && lane < 32))
                direct_load16(Vw + chn * NVEC * CH + 4 * (64 * hw + lane),
                              B + L::OFF_VEC + 1024 * hw);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        };
        stage(0, 0);
        lds_barrier();
        for (int c = 0; c < NC; ++c) {
            if (c + 1 < NC) stage(c + 1, (c + 1) & 1);
            lds_barrier();
        }
        return;
    }

    // ---------------- compute wavefronts ----------------
    const int wl = 16 * wave + l16;            // this lane's column inside the tile
    const int col = tile * TV + wl;            // ... inside the head

    // state slots: S[phys_row(16 rt + 4 lg + r)][col]
    f32x4 Sa[RT], Ma[RT];
    const size_t sbase = (size_t)bh * DK * DV;
    auto load_state = [&](f32x4* X, const float* src) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                X[rt][r] = src ? src[sbase + (size_t)phys_row(16 * rt + 4 * lg + r) * DV + col] : 0.f;
    };
    if (S0) load_state(Sa, S0); else load_state(Sa, nullptr);
    if (M0) load_state(Ma, M0); else load_state(Ma, nullptr);

    // per-lane fragment row bases (bytes), the same every chunk
    int kq_base[4], c_base[4], v_off[4], orow[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int r = phys_row(16 * x + l16);
        kq_base[x] = LK::chunk(r, lg);
        c_base[x] = LC::chunk(r, lg);
        orow[x] = r;
        // V rows phys_row(16 x + 4 lg) + j, columns 16 w + 4 m .. + 3 (lane
        // 4 j + m of its group): the transposing read hands lane l16 column
        // 16 w + l16 of those four rows
        const int c4 = 16 * wave + 4 * (l16 & 3);
        v_off[x] = L::OFF_V + LC::chunk(phys_row(16 * x + 4 * lg) + (l16 >> 2), c4 >> 3) +
                   2 * (c4 & 7);
    }
    // K^T fragments of the update (tile rt, half hf, step s): lane 4 j + m of
    // group lg reads K row 32 s + 8 lg + 4 hf + j, columns
    // phys_row(16 rt + 4 m) .. + 3; the transposing read hands lane l16
    // column phys_row(16 rt + l16) of those four rows.  Rows 32 s + x lie
    // L::KSTEP_ROWS bytes after row x.
    int kt_off[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            kt_off[rt][hf] = LK::chunk(8 * lg + 4 * hf + (l16 >> 2), 4 * (rt >> 1) + (l16 & 3)) +
                             8 * (rt & 1);
    const unsigned ostride = (unsigned)(H * DV);
    E* const Ocol = O + ((size_t)b * T * H + h) * DV + tile * TV + 16 * wave + 4 * lg;

    lds_barrier();                           // chunk 0 staged
    for (int c = 0; c < NC; ++c) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const char* Kb = buf[c & 1];
        const char* Qb = Kb + L::OFF_Q;
        const char* Tb = Kb + L::OFF_T;
        const char* Ab = Kb + L::OFF_A;
        const float* vec = reinterpret_cast<const float*>(Kb + L::OFF_VEC);

        // (1) X = K [S | M]: the critical path first (the state update below
        //     needs Vt, which needs R, which needs X)
        f32x4 R[4];
        {
            f32x4 xs[4], xm[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) xs[ct] = xm[ct] = zero4();
            bf16x8 aK[SK][4];
#pragma unroll
            for (int s = 0; s < SK; ++s)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    aK[s][ct] = *reinterpret_cast<const bf16x8*>(Kb + kq_base[ct] + 64 * s);
#pragma unroll
            for (int s = 0; s < SK; ++s) {
                const auto bS = MM::from_acc(Sa, s);
                const auto bM = MM::from_acc(Ma, s);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    xs[ct] = MM::mma(aK[s][ct], bS, xs[ct]);
                    xm[ct] = MM::mma(aK[s][ct], bM, xm[ct]);
                }
            }
            // (2) R = V - Diag(abar) K S0 + Diag(alpha b^-) K M0; slot (ct, lg, r)
            //     is chunk row phys_row(16 ct + 4 lg + r), four consecutive rows
            //     per (ct, lg), which V^T holds contiguously
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int p0 = phys_row(16 * ct + 4 * lg);
                const f32x4 ab = *reinterpret_cast<const f32x4*>(vec + V_ABAR * CH + p0);
                const f32x4 ab1 = *reinterpret_cast<const f32x4*>(vec + V_AB1 * CH + p0);
                const bf16x4 vv = lds_read_tr4(Kb + v_off[ct]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    R[ct][r] = static_cast<float>(vv[r]) - ab[r] * xs[ct][r] + ab1[r] * xm[ct][r];
            }
        }

        // (3) Vt = T R
        f32x4 Vt[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) Vt[it] = zero4();
#pragma unroll
        for (int s = 0; s < SC; ++s) {
            const auto bR = MM::from_acc(R, s);
#pragma unroll
            for (int it = 0; it < 4; ++it)
                Vt[it] = MM::mma(*reinterpret_cast<const bf16x8*>(Tb + c_base[it] + 64 * s), bR,
                                 Vt[it]);
        }

        // (4) O^T = S0^T Q^T Diag(abar) - M0^T Q^T Diag(b) + Vt^T A^T (from the
        //     entry state); lane: output row orow[ct], columns 4 lg .. + 3
        f32x4 Ot[4];
        {
            f32x4 ys[4], ym[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) ys[ct] = ym[ct] = zero4();
            bf16x8 aQ[SK][4];
#pragma unroll
            for (int s = 0; s < SK; ++s)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    aQ[s][ct] = *reinterpret_cast<const bf16x8*>(Qb + kq_base[ct] + 64 * s);
#pragma unroll
            for (int s = 0; s < SK; ++s) {
                const auto bS = MM::from_acc(Sa, s);
                const auto bM = MM::from_acc(Ma, s);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    ys[ct] = MM::mma(bS, aQ[s][ct], ys[ct]);
                    ym[ct] = MM::mma(bM, aQ[s][ct], ym[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const float ab = vec[V_ABAR * CH + orow[ct]];
                const float bb = vec[V_B * CH + orow[ct]];
                Ot[ct] = ab * ys[ct] - bb * ym[ct];
            }
        }
#pragma unroll
        for (int s = 0; s < SC; ++s) {
            const auto aV = MM::from_acc(Vt, s);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                Ot[ct] = MM::mma(aV, *reinterpret_cast<const bf16x8*>(Ab + c_base[ct] + 64 * s),
                                 Ot[ct]);
        }
        {
            E* Ob = Ocol + (size_t)t0 * ostride;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                if (orow[ct] < n)
                    store4<E>(Ob + (unsigned)orow[ct] * ostride, Ot[ct][0], Ot[ct][1], Ot[ct][2],
                              Ot[ct][3]);
        }

        // (5) S' = abar_n S0 - b_n M0 + K^T Diag(eta gamma_n) Vt,
        //     M' = mubar_n M0 - K^T Diag(eta mubar_n / mubar) Vt
        const float abn = vec[V_SCAL * CH + 0];
        const float bn = vec[V_SCAL * CH + 1];
        const float mbn = vec[V_SCAL * CH + 2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            Sa[rt] = abn * Sa[rt] - bn * Ma[rt];
            Ma[rt] = mbn * Ma[rt];
        }
#pragma unroll
        for (int s = 0; s < SC; ++s) {
            const auto bS = MM::from_acc_scaled8(Vt, s, vec + V_WS * CH + 32 * s + 8 * lg, 1.f);
            const auto bM = MM::from_acc_scaled8(Vt, s, vec + V_WM * CH + 32 * s + 8 * lg, -1.f);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const bf16x4 lo = lds_read_tr4(Kb + kt_off[rt][0] + s * L::KSTEP_ROWS);
                const bf16x4 hi = lds_read_tr4(Kb + kt_off[rt][1] + s * L::KSTEP_ROWS);
                const bf16x8 aK = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                Sa[rt] = MM::mma(aK, bS, Sa[rt]);
                Ma[rt] = MM::mma(aK, bM, Ma[rt]);
            }
        }
        // this chunk's buffer is free and the next one is staged
        lds_barrier();
    }

    auto store_state = [&](float* dst, const f32x4* X) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[sbase + (size_t)phys_row(16 * rt + 4 * lg + r) * DV + col] = X[rt][r];
    };
    if (ST) store_state(ST, Sa);
    if (MT) store_state(MT, Ma);
}

// ---------------------------------------------------------------------------
// bf16 scan for layers with few heads ("row split").  When B * H * DV / 64 is
// well below the number of compute units, one workgroup per 64 value columns
// leaves most of the chip idle, and each chunk costs the latency of one
// wavefront's whole chain (K S, the substitution, the outputs, the update of
// all DK state rows).  Here a workgroup owns 16 value columns, and its NW
// compute wavefronts split the state rows: wavefront w holds rows
// [RW w, RW w + RW), RW = DK / NW, of S and M for those columns, for the
// whole sequence.  The chunk equations are those of chunk_scan_bf16_kernel;
// per chunk:
//   (a) products over the wavefront's own rows: K_w [S_w | M_w] gives its
//       share of R = V - Diag(abar) K S0 + Diag(alpha b^-) K M0 (wavefront 0
//       adds V), and [S_w | M_w]^T Q_w^T its share of the outputs' entry-state
//       part; the shares go to LDS (each wavefront keeps its own);
//   barrier;
//   (b) every wavefront sums the R shares and forms all of Vt = T R (the same
//       8 products on each wavefront, cheaper than a second exchange),
//       updates its rows with K_w^T Diag(w) Vt, and finishes the output rows
//       of its own 16-row tiles (the sum of the shares plus Vt^T A^T);
//   barrier.
// Four staging wavefronts bring chunk c + 1 into the other buffer
// meanwhile, with direct global-to-LDS loads only: the transposed K of the
// update and V in the layout of R are read from the row-major tiles with
// transposing LDS reads.  The 16-column strips of one head run on one XCD,
// so the head's K, Q, T and A come from HBM once and from that L2 after.
// MU = false is the momentum-free case (mu = 0: b, alpha b^- and mubar_n
// vanish, so M never feeds S): every product with M is dropped, M0 is not
// read, and M_T is formed in the last chunk only, from the zero momentum.
// ---------------------------------------------------------------------------
template <int DK, int NW>
struct ScanRsLayout {
    using LK = TileLayout<DK * 2>;          // K, Q rows
    using LC = TileLayout<CH * 2>;          // T, A rows
    static constexpr int RW = DK / NW;      // state rows per compute wavefront
    static constexpr int NS = 4;            // staging wavefronts
    static constexpr int TS = 16;           // value columns per workgroup
    static_assert(RW == 32 || RW == 64, "rows per wavefront");
    static constexpr int OFF_Q = LK::BYTES;
    static constexpr int OFF_T = 2 * LK::BYTES;
    static constexpr int OFF_A = OFF_T + LC::BYTES;
    static constexpr int OFF_V = OFF_A + LC::BYTES;     // 64 rows x 32 bytes, row-major
    static constexpr int OFF_VEC = OFF_V + CH * TS * 2;
    static constexpr int BUF_BYTES = OFF_VEC + 6 * CH * 4;
    // one f32x4 per (wavefront, 16-row tile, lane)
    static constexpr int SHARE_BYTES = NW * 4 * 64 * 16;
    static constexpr int OFF_RP = 2 * BUF_BYTES;
    static constexpr int OFF_OP = OFF_RP + SHARE_BYTES;
    static constexpr int BYTES = OFF_OP + SHARE_BYTES;
    // byte distance between the rows 32 s + x and x of a K tile
    static constexpr int KSTEP_ROWS = 32 * (DK * 2) + (32 / LK::G) * LK::PAD;
    static_assert(BYTES <= 160 * 1024, "LDS");
};

// The LDS buffer index of a chunk: a compile-time constant when the chunk
// loop is unrolled by two, a run-time parity otherwise.
template <int V>
__device__ constexpr int buf_of(std::integral_constant<int, V>) { return V; }
__device__ inline int buf_of(int b) { return b; }

template <int DK, int DV, int NW, bool UNROLL, bool MU>
__global__ __launch_bounds__(64 * (NW + 4)) void chunk_scan_rs_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ Tw, const __bf16* __restrict__ Aw, const float* __restrict__ Vw,
    const float* S0, const float* M0, __bf16* __restrict__ O, float* ST, float* MT, int T, int H,
    int NC, int xcd_groups)
{
    using E = __bf16;
    using MM = Mma<E>;
    using L = ScanRsLayout<DK, NW>;
    using LK = typename L::LK;
    using LC = typename L::LC;
    constexpr int RW = L::RW;
    constexpr int RT = RW / 16;             // state row tiles per wavefront
    constexpr int SKW = RW / 32;            // k-steps of the shares
    constexpr int TS = L::TS;
    constexpr int NSTRIP = DV / TS;
    constexpr int CTW = 4 / NW;             // output row tiles each compute wavefront finishes

    __shared__ __align__(16) char smem[L::BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;

    unsigned bid = blockIdx.x;
    if (xcd_groups > 0) bid = (bid % 8u) * (unsigned)xcd_groups + bid / 8u;
    const int strip = (int)(bid % NSTRIP);
    const int bh = (int)(bid / NSTRIP);
    const int h = bh % H;
    const int b = bh / H;
    const size_t tokb = (size_t)b * T * H + h;   // token (b, 0, h)

    if (wave >= NW) {
        // ---------------- staging wavefronts ----------------
        const int hw = wave - NW;
        const unsigned kq_stride = (unsigned)(H * DK);
        const unsigned kq_lane = LK::lane_offset(kq_stride, lane);
        const unsigned c_lane = LC::lane_offset(CH, lane);
        auto stage = [&](int c, int bi) {
            const int n = min(CH, T - c * CH);
            const size_t tok0 = tokb + (size_t)c * CH * H;
            const size_t chn = (size_t)bh * NC + c;
            char* B = smem + bi * L::BUF_BYTES;
            LK::load(B, k + tok0 * DK, kq_stride, kq_lane, n, hw, lane);
            LK::load(B + L::OFF_Q, q + tok0 * DK, kq_stride, kq_lane, n, hw, lane);
            LC::load(B + L::OFF_T, Tw + chn * CH * CH, CH, c_lane, CH, hw, lane);
            LC::load(B + L::OFF_A, Aw + chn * CH * CH, CH, c_lane, CH, hw, lane);
            if (hw < 2) {
                // the strip of V: lane l brings half l % 2 of row 32 hw + l / 2
                // (rows >= n read row n - 1)
                const int row = min(32 * hw + (lane >> 1), n - 1);
                direct_load16(v + (tok0 + (size_t)row * H) * DV + strip * TS + 8 * (lane & 1),
                              B + L::OFF_V + 1024 * hw);
            } else if (hw == 2 || lane < 32) {
                // coefficient vectors: 6 x 64 floats = 96 pieces of 16 bytes
                direct_load16(Vw + chn * NVEC * CH + 4 * (64 * (hw - 2) + lane),
                              B + L::OFF_VEC + 1024 * (hw - 2));
            }
        };
        stage(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        for (int c = 0; c < NC; ++c) {
            if (c + 1 < NC) stage(c + 1, (c + 1) & 1);
            lds_barrier();                                   // (a) -> (b)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();                                   // chunk c + 1 staged
        }
        return;
    }

    // ---------------- compute wavefronts ----------------
    const int w = wave;
    const int col = strip * TS + l16;                       // this lane's state column

    // state slot (rt, lg, r): row RW w + phys_row(16 rt + 4 lg + r), column col
    f32x4 Sa[RT], Ma[RT];
    const size_t sbase = (size_t)bh * DK * DV;
    auto srow = [&](int rt, int r) { return RW * w + phys_row(16 * rt + 4 * lg + r); };
    auto load_state = [&](f32x4* X, const float* src) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                X[rt][r] = src ? src[sbase + (size_t)srow(rt, r) * DV + col] : 0.f;
    };
    if (S0) load_state(Sa, S0); else load_state(Sa, nullptr);
    if (MU && M0) load_state(Ma, M0); else load_state(Ma, nullptr);

    // per-lane LDS byte offsets, the same every chunk
    int kq_base[4], c_base[4], v_off[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int r = phys_row(16 * x + l16);
        // K_w / Q_w fragment of step s: row r, columns RW w + 32 s + 8 lg .. + 7
        kq_base[x] = LK::chunk(r, (RW / 8) * w + lg);
        c_base[x] = LC::chunk(r, lg);
        // V rows phys_row(16 x + 4 lg) + j, columns 4 m .. + 3 (lane 4 j + m
        // of its group): the transposing read hands lane l16 column l16
        v_off[x] = L::OFF_V + (phys_row(16 * x + 4 * lg) + (l16 >> 2)) * (TS * 2) + 8 * (l16 & 3);
    }
    // The output row tiles in this wavefront's order: tile j is
    // ct_j = (CTW w + j) mod 4, so that its own tiles (those it finishes) are
    // j < CTW.  Everything indexed by ct_j is a per-lane constant, chosen
    // here once, so the chunk loop has no wavefront-dependent branches.
    int q_rot[4], a_rot[4], orow_rot[4], op_rot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ctj = (CTW * w + j) & 3;
        const int r = phys_row(16 * ctj + l16);
        q_rot[j] = LK::chunk(r, (RW / 8) * w + lg);
        a_rot[j] = LC::chunk(r, lg);
        orow_rot[j] = r;
        op_rot[j] = ((w * 4 + ctj) * 64 + lane) * 16;             // this wavefront's share
    }
    // K_w^T fragments of the update (tile rt, half hf, step s): lane 4 j + m
    // of group lg reads K row 32 s + 8 lg + 4 hf + j, columns
    // RW w + phys_row(16 rt + 4 m) .. + 3; the transposing read hands lane l16
    // column RW w + phys_row(16 rt + l16) of those four rows.  Rows 32 s + x
    // lie L::KSTEP_ROWS bytes after row x.
    int kt_off[RT][2];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            kt_off[rt][hf] = LK::chunk(8 * lg + 4 * hf + (l16 >> 2),
                                       (RW / 8) * w + 4 * (rt >> 1) + (l16 & 3)) + 8 * (rt & 1);
    // the other wavefronts' shares, in the order w + 1, w + 2, ... (mod NW)
    int peer[NW > 1 ? NW - 1 : 1];
#pragma unroll
    for (int u = 1; u < NW; ++u) peer[u - 1] = (w + u) % NW;
    const float vsel = w == 0 ? 1.f : 0.f;                  // wavefront 0 adds V to its share
    const unsigned ostride = (unsigned)(H * DV);
    E* const Ocol = O + tokb * DV + strip * TS + 4 * lg;
    char* const Rp = smem + L::OFF_RP;
    char* const Op = smem + L::OFF_OP;
    auto share = [](char* base, int off) -> f32x4& { return *reinterpret_cast<f32x4*>(base + off); };

    // one chunk; `bi` is its LDS buffer (chunk c sits in buffer c mod 2)
    auto chunk_step = [&](const int c, auto bi) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const char* Kb = smem + buf_of(bi) * L::BUF_BYTES;
        const char* Qb = Kb + L::OFF_Q;
        const char* Tb = Kb + L::OFF_T;
        const char* Ab = Kb + L::OFF_A;
        const float* vec = reinterpret_cast<const float*>(Kb + L::OFF_VEC);

        // (a) shares over this wavefront's rows.  Operands are read in the
        //     order they are needed: K first (the critical path), then what
        //     the rest of the chunk reads from this buffer, so that those
        //     reads overlap the products instead of following the exchange.
        //     T is lower triangular by 16-row blocks: its upper right 32 x 32
        //     block is neither read nor multiplied.
        bf16x8 aK[SKW][4];
#pragma unroll
        for (int s = 0; s < SKW; ++s)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                aK[s][ct] = *reinterpret_cast<const bf16x8*>(Kb + kq_base[ct] + 64 * s);
        f32x4 ab[4], ab1[4];
        bf16x4 vv[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int p0 = phys_row(16 * ct + 4 * lg);
            ab[ct] = *reinterpret_cast<const f32x4*>(vec + V_ABAR * CH + p0);
            if (MU) ab1[ct] = *reinterpret_cast<const f32x4*>(vec + V_AB1 * CH + p0);
            vv[ct] = lds_read_tr4(Kb + v_off[ct]);
        }
        bf16x8 aQ[SKW][4], aT[2][4], aA[2][CTW];
        bf16x4 kt[2][RT][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int it = 2 * s; it < 4; ++it)
                aT[s][it] = *reinterpret_cast<const bf16x8*>(Tb + c_base[it] + 64 * s);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                    kt[s][rt][hf] = lds_read_tr4(Kb + kt_off[rt][hf] + s * L::KSTEP_ROWS);
        }
#pragma unroll
        for (int s = 0; s < SKW; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                aQ[s][j] = *reinterpret_cast<const bf16x8*>(Qb + q_rot[j] + 64 * s);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int u = 0; u < CTW; ++u)
                aA[s][u] = *reinterpret_cast<const bf16x8*>(Ab + a_rot[u] + 64 * s);

        f32x4 rown[4], oown[CTW];
        {
            f32x4 xs[4], xm[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) xs[ct] = xm[ct] = zero4();
#pragma unroll
            for (int s = 0; s < SKW; ++s) {
                const auto bS = MM::from_acc(Sa, s);
                const auto bM = MM::from_acc(Ma, s);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    xs[ct] = MM::mma(aK[s][ct], bS, xs[ct]);
                    if (MU) xm[ct] = MM::mma(aK[s][ct], bM, xm[ct]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                f32x4 rp;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    rp[r] = vsel * static_cast<float>(vv[ct][r]) - ab[ct][r] * xs[ct][r];
                    if (MU) rp[r] += ab1[ct][r] * xm[ct][r];
                }
                rown[ct] = rp;
                share(Rp, ((w * 4 + ct) * 64 + lane) * 16) = rp;
            }
        }
        {
            f32x4 ys[4], ym[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) ys[j] = ym[j] = zero4();
#pragma unroll
            for (int s = 0; s < SKW; ++s) {
                const auto bS = MM::from_acc(Sa, s);
                const auto bM = MM::from_acc(Ma, s);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ys[j] = MM::mma(bS, aQ[s][j], ys[j]);
                    if (MU) ym[j] = MM::mma(bM, aQ[s][j], ym[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 op = vec[V_ABAR * CH + orow_rot[j]] * ys[j];
                if (MU) op -= vec[V_B * CH + orow_rot[j]] * ym[j];
                if (j < CTW) oown[j] = op;
                else share(Op, op_rot[j]) = op;
            }
        }
        lds_barrier();

        // (b) R, Vt = T R
        f32x4 R[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            R[ct] = rown[ct];
#pragma unroll
            for (int u = 0; u < NW - 1; ++u)
                R[ct] += share(Rp, ((peer[u] * 4 + ct) * 64 + lane) * 16);
        }
        f32x4 Vt[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) Vt[it] = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const auto bR = MM::from_acc(R, s);
#pragma unroll
            for (int it = 2 * s; it < 4; ++it) Vt[it] = MM::mma(aT[s][it], bR, Vt[it]);
        }

        // S' = abar_n S0 - b_n M0 + K^T Diag(eta gamma_n) Vt,
        // M' = mubar_n M0 - K^T Diag(eta mubar_n / mubar) Vt, on this wavefront's rows
        const float abn = vec[V_SCAL * CH + 0];
        const float bn = vec[V_SCAL * CH + 1];
        const float mbn = vec[V_SCAL * CH + 2];
        // without momentum M' matters only after the last chunk
        const bool upd_m = MU || (MT != nullptr && c == NC - 1);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (MU) {
                Sa[rt] = abn * Sa[rt] - bn * Ma[rt];
                Ma[rt] = mbn * Ma[rt];
            } else {
                Sa[rt] = abn * Sa[rt];
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const auto bS = MM::from_acc_scaled8(Vt, s, vec + V_WS * CH + 32 * s + 8 * lg, 1.f);
            const auto bM = MM::from_acc_scaled8(Vt, s, vec + V_WM * CH + 32 * s + 8 * lg, -1.f);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const bf16x4 lo = kt[s][rt][0], hi = kt[s][rt][1];
                const bf16x8 aKt = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                Sa[rt] = MM::mma(aKt, bS, Sa[rt]);
                if (upd_m) Ma[rt] = MM::mma(aKt, bM, Ma[rt]);
            }
        }

        // outputs of this wavefront's row tiles: O^T = sum of the shares + Vt^T A^T
#pragma unroll
        for (int u = 0; u < CTW; ++u) {
            f32x4 ot = oown[u];
            // the share of wavefront x for this tile sits (x - w) * 4 KB from ours
#pragma unroll
            for (int x = 0; x < NW - 1; ++x)
                ot += share(Op, op_rot[u] + (peer[x] - w) * 4 * 64 * 16);
#pragma unroll
            for (int s = 0; s < 2; ++s) ot = MM::mma(MM::from_acc(Vt, s), aA[s][u], ot);
            if (orow_rot[u] < n)
                store4<E>(Ocol + (size_t)(t0 + orow_rot[u]) * ostride, ot[0], ot[1], ot[2], ot[3]);
        }
        // this chunk's buffer and the shares are free; the next chunk is staged
        lds_barrier();
    };
    lds_barrier();                                          // chunk 0 staged
    if constexpr (UNROLL) {
        // two chunks per iteration: every LDS address is a per-lane base
        // plus an immediate
        for (int c = 0; c < NC; c += 2) {
            chunk_step(c, std::integral_constant<int, 0>{});
            if (c + 1 < NC) chunk_step(c + 1, std::integral_constant<int, 1>{});
        }
    } else {
        for (int c = 0; c < NC; ++c) chunk_step(c, c & 1);
    }

    auto store_state = [&](float* dst, const f32x4* X) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[sbase + (size_t)srow(rt, r) * DV + col] = X[rt][r];
    };
    if (ST) store_state(ST, Sa);
    if (MT) store_state(MT, Ma);
}

// T = 0: the final state is the initial state (zero when absent)
__global__ __launch_bounds__(NT) void state_passthrough_kernel(const float* __restrict__ src,
                                                               float* dst, size_t count)
{
    const size_t i = (size_t)blockIdx.x * NT + threadIdx.x;
    if (i < count) dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <typename E, int DK>
static hipError_t launch_prepare_t(const void* q, const void* k, const float* alpha,
                                   const float* mu, const float* eta, const float* beta, int B,
                                   int T, int H, void* workspace, hipStream_t stream)
{
    const int NC = (T + CH - 1) / CH;
    const size_t nchunks = (size_t)B * H * NC;
    Workspace<E> ws = ws_carve<E>(workspace, nchunks);
    hipLaunchKernelGGL((chunk_prep_kernel<E, DK>), dim3((unsigned)nchunks), dim3(NT), 0, stream,
                       static_cast<const E*>(q), static_cast<const E*>(k), alpha, mu, eta, beta,
                       ws.T, ws.A, ws.vec, T, H, NC);
    return hipGetLastError();
}

template <typename E, int DK, int DV>
static hipError_t launch_scan_t(const void* q, const void* k, const void* v, const float* S0,
                                const float* M0, void* O, void* Vto, float* ST, float* MT, int B,
                                int T, int H, const void* workspace, hipStream_t stream)
{
    const int NC = (T + CH - 1) / CH;
    const size_t nchunks = (size_t)B * H * NC;
    Workspace<E> ws = ws_carve<E>(const_cast<void*>(workspace), nchunks);
    const size_t nblk = (size_t)B * H * (DV / ScanSmem<E, DK, DV>::TV);
    const int xcd_groups = nblk % 8 == 0 ? (int)(nblk / 8) : 0;
    if (sizeof(E) == 2 && Vto) return hipErrorInvalidValue;   // not stored by this path
    if constexpr (sizeof(E) == 2) {
        hipLaunchKernelGGL((chunk_scan_bf16_kernel<DK, DV>), dim3((unsigned)nblk), dim3(2 * NT), 0,
                           stream, static_cast<const E*>(q), static_cast<const E*>(k),
                           static_cast<const E*>(v), ws.T, ws.A, ws.vec, S0, M0,
                           static_cast<E*>(O), ST, MT, T, H, NC, xcd_groups);
    } else {
        hipLaunchKernelGGL((chunk_scan_kernel<E, DK, DV>), dim3((unsigned)nblk), dim3(NT), 0,
                           stream, static_cast<const E*>(q), static_cast<const E*>(k),
                           static_cast<const E*>(v), ws.T, ws.A, ws.vec, S0, M0,
                           static_cast<E*>(O), static_cast<E*>(Vto), ST, MT, T, H, NC,
                           xcd_groups);
    }
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_scan_rs_t(const void* q, const void* k, const void* v, const float* S0,
                                   const float* M0, void* O, float* ST, float* MT, int B, int T,
                                   int H, bool momentum, const void* workspace,
                                   hipStream_t stream)
{
    // Compute wavefronts per strip and loop shape, as measured fastest at
    // B1 H16 T16384 d128: with momentum four wavefronts (32 rows each) and the
    // loop unrolled by two; without, two wavefronts (64 rows each; unrolled,
    // their registers would spill).  Dk = 64 always runs two.
    constexpr int NW = DK == 64 ? 2 : 4;
    using L = ScanRsLayout<DK, NW>;
    using L2 = ScanRsLayout<DK, 2>;
    const int NC = (T + CH - 1) / CH;
    const size_t nchunks = (size_t)B * H * NC;
    Workspace<__bf16> ws = ws_carve<__bf16>(const_cast<void*>(workspace), nchunks);
    const size_t nblk = (size_t)B * H * (DV / L::TS);
    if (nblk > 0xffffffffu) return hipErrorInvalidValue;
    const int xcd_groups = nblk % 8 == 0 ? (int)(nblk / 8) : 0;
    auto kern = momentum ? chunk_scan_rs_kernel<DK, DV, NW, DK != 64, true>
                         : chunk_scan_rs_kernel<DK, DV, 2, false, false>;
    const int waves = momentum ? NW + L::NS : 2 + L2::NS;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(64 * waves), 0, stream,
                       static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                       static_cast<const __bf16*>(v), ws.T, ws.A, ws.vec, S0, M0,
                       static_cast<__bf16*>(O), ST, MT, T, H, NC, xcd_groups);
    return hipGetLastError();
}

// dst = src (src NULL: zero), count floats
hipError_t launch_state_copy(const float* src, float* dst, size_t count, hipStream_t stream)
{
    if (count == 0) return hipSuccess;
    const unsigned grid = (unsigned)((count + NT - 1) / NT);
    hipLaunchKernelGGL(state_passthrough_kernel, dim3(grid), dim3(NT), 0, stream, src, dst, count);
    return hipGetLastError();
}

size_t chunk_workspace_bytes(int B, int T, int H, bool bf16)
{
    const size_t NC = ((size_t)T + CH - 1) / CH;
    const size_t nchunks = (size_t)B * H * NC;
    return bf16 ? ws_bytes<__bf16>(nchunks) : ws_bytes<float>(nchunks);
}

hipError_t launch_chunk_prepare(const void* q, const void* k, const float* alpha, const float* mu,
                                const float* eta, const float* beta, int B, int T, int H, int Dk,
                                bool bf16, void* workspace, hipStream_t stream)
{
    if (T == 0) return hipSuccess;
#define MDN_PREP(E, DK)                                                                          \
    if (Dk == DK)                                                                                \
        return launch_prepare_t<E, DK>(q, k, alpha, mu, eta, beta, B, T, H, workspace, stream);
    if (bf16) {
        MDN_PREP(__bf16, 64) MDN_PREP(__bf16, 128)
    } else {
        MDN_PREP(float, 64) MDN_PREP(float, 128)
    }
#undef MDN_PREP
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_scan(const void* q, const void* k, const void* v, const float* S0,
                             const float* M0, void* O, void* Vto, float* ST, float* MT, int B,
                             int T, int H, int Dk, int Dv, bool bf16, bool row_split,
                             bool momentum, const void* workspace, hipStream_t stream)
{
    if (T == 0) {
        const size_t count = (size_t)B * H * Dk * Dv;
        const unsigned grid = (unsigned)((count + NT - 1) / NT);
        if (ST) {
            hipLaunchKernelGGL(state_passthrough_kernel, dim3(grid), dim3(NT), 0, stream, S0, ST,
                               count);
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
        if (MT) {
            hipLaunchKernelGGL(state_passthrough_kernel, dim3(grid), dim3(NT), 0, stream, M0, MT,
                               count);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    if (bf16 && row_split) {
        if (Vto) return hipErrorInvalidValue;   // the row-split scan does not store Vt
#define MDN_SCAN_RS(DK, DV)                                                                      \
    if (Dk == DK && Dv == DV)                                                                    \
        return launch_scan_rs_t<DK, DV>(q, k, v, S0, M0, O, ST, MT, B, T, H, momentum,      \
                                        workspace, stream);
        MDN_SCAN_RS(64, 64) MDN_SCAN_RS(64, 128) MDN_SCAN_RS(128, 64) MDN_SCAN_RS(128, 128)
#undef MDN_SCAN_RS
        return hipErrorInvalidValue;
    }
#define MDN_SCAN(E, DK, DV)                                                                      \
    if (Dk == DK && Dv == DV)                                                                    \
        return launch_scan_t<E, DK, DV>(q, k, v, S0, M0, O, Vto, ST, MT, B, T, H, workspace, stream);
    if (bf16) {
        MDN_SCAN(__bf16, 64, 64) MDN_SCAN(__bf16, 64, 128)
        MDN_SCAN(__bf16, 128, 64) MDN_SCAN(__bf16, 128, 128)
    } else {
        MDN_SCAN(float, 64, 64) MDN_SCAN(float, 64, 128)
        MDN_SCAN(float, 128, 64) MDN_SCAN(float, 128, 128)
    }
#undef MDN_SCAN
    return hipErrorInvalidValue;
}

}  // namespace mdn
