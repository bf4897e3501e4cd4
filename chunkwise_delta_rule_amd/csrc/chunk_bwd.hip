// chunk_bwd.hip -- chunkwise MDN backward pass on gfx950.
//
// The pages ("MDN: Parallelizing Stepwise Momentum for Delta Linear
// Attention" (slides), frame "The implementation trades saved residuals for
// throughput"; the reading notes on the same paper, Sec. 2.6) give the
// backward pass's strategy -- keep the residuals Vt, rebuild the states from
// them, store no full state pair per chunk between the passes -- but no
// gradient formulas.  The formulas below are the chain rule applied to the
// chunk equations of the forward (chunk_fwd.hip), per chunk of C = 64 tokens
// with entry state (S0, M0), exit-state gradients (dS', dM') and the same
// coefficients (abar, b, ab1_i = alpha_i b_{i-1}, Gamma, m, ws = eta o
// Gamma_{n,:}, wm = eta o m_{n,:}; P = Diag(alpha) K, Khat = Diag(eta) K):
//
//   dVt  = A^T dO + Diag(ws) K dS' - Diag(wm) K dM'
//   dR   = T^T dVt                                  (= dV)
//   dS0  = abar_n dS' + Q^T Diag(abar) dO - K^T Diag(abar) dR
//   dM0  = mubar_n dM' - b_n dS' - Q^T Diag(b) dO + K^T Diag(ab1) dR
//   dA   = tril(dO Vt^T),  dL = -stril(dR Vt^T)
//   dQ   = Diag(abar) dO S0^T - Diag(b) dO M0^T + (dA o Gamma) Khat
//   dKhat = (dA o Gamma)^T Q + (dL o Gamma^-)^T P,  dP = (dL o Gamma^-) Khat
//   dK   = Diag(eta) dKhat + Diag(alpha) dP - Diag(abar) dR S0^T + Diag(ab1) dR M0^T
//          + Diag(ws) Vt dS'^T - Diag(wm) Vt dM'^T
// and, for the gates, the gradients of the coefficients
//   dabar_i = q_i.(dO S0^T)_i - k_i.(dR S0^T)_i,  db_i = -q_i.(dO M0^T)_i,
//   d(ab1)_i = k_i.(dR M0^T)_i,  plus <dS', S0>, -<dS', M0>, <dM', M0> on the
//   last row's abar_n, b_n, mubar_n;
//   dGamma = dA o (Q Khat^T) + (dL o (P Khat^T)) shifted up one row, plus
//   eta_j k_j.(Vt dS'^T)_j on the last row;  dm_{n,j} = -eta_j k_j.(Vt dM'^T)_j
// carried back through the coefficient recursions (abar_i = alpha_i abar_{i-1},
// mubar_i = mu_i mubar_{i-1}, b_i = alpha_i b_{i-1} + beta_i mubar_i,
// gamma_{i,j} = alpha_i gamma_{i-1,j} + beta_i m_{i,j}, m_{i,j} = mu_i m_{i-1,j})
// and the direct uses of eta (Khat, ws, wm) and alpha (P, ab1).
//
// Given the residuals Vt that the forward saved, the re-scan below rebuilds
// the chunk-entry states from them with no solve; given none, it runs the
// forward's solve again.  Each chunk's entry state and exit-state gradients
// are kept in the workspace (in the I/O type) only while the call runs.
//
// Kernels, in launch order (after chunk_prep_kernel has written T, A and the
// coefficient rows of every chunk):
//   reverse scan        one workgroup per (b, h, 64 value columns), chunks last
//                       to first: dVt, dR (written as dv), the state gradients
//                       carried back, and each chunk's exit-state gradients
//                       stored for the last kernel (bwd_scan_kernel for fp32
//                       I/O; bwd_scan_bf16_kernel, with staging wavefronts and
//                       bf16 tiles, for bf16 I/O).
//   re-scan             the same grid, chunks first to last: the state update
//                       again (with R and Vt = T R unless Vt was saved),
//                       storing each chunk's entry state (and Vt)
//                       (bwd_rescan_kernel; bwd_rescan_bf16_kernel).
//   per-chunk products  one workgroup per chunk, all columns: dq, dk and the
//                       gate gradients (bwd_grad_kernel; bwd_grad_bf16_kernel).
// Arithmetic is fp32 (v_mfma_f32_16x16x4_f32 and VALU; bf16 inputs are
// widened when they are staged into LDS), except that with bf16 I/O the two
// scans run all their products on v_mfma_f32_16x16x32_bf16 (each kernel
// states which operands are exact in bf16, which are rounded and which are
// split into two bf16 parts), and bwd_grad_bf16_kernel runs the six products
// of a row operand with a stored bf16 state (the row operand rounded to bf16:
// exact for dO and for saved Vt), the chunk products dO Vt^T, K K^T and Q K^T
// (exact operands, but for a recomputed Vt) and the masked products (head
// and remainder operands) on it.
#include <hip/hip_runtime.h>

#include "chunk_common.hpp"
#include "mfma.hpp"

namespace mdn {

hipError_t launch_chunk_prepare(const void* q, const void* k, const float* alpha, const float* mu,
                                const float* eta, const float* beta, int B, int T, int H, int Dk,
                                bool bf16, void* workspace, hipStream_t stream);

namespace {

using MF = Mma<float>;

__device__ __forceinline__ float ldf(const float* p) { return *p; }
__device__ __forceinline__ float ldf(const __bf16* p) { return static_cast<float>(*p); }

// A C x D tile of a row-major array (row stride in elements) on its way to
// fp32 LDS with row stride LD: fetch() issues every 16-byte load of this
// thread into registers (rows >= n read as zero), commit() widens and stores
// them, so that the loads of several tiles (or of the next chunk) are in
// flight together.
template <typename E, int D, int LD>
struct Tile {
    static constexpr int VE = 16 / sizeof(E);    // elements per load
    static constexpr int VPR = D / VE;           // loads per row
    static constexpr int NV = CH * VPR / NT;     // loads per thread
    static_assert(CH * VPR % NT == 0, "tile must split evenly over the workgroup");
    uint4 buf[NV];
    __device__ __forceinline__ void fetch(const E* __restrict__ src, size_t stride, int n, int tid)
    {
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int idx = tid + u * NT;
            const int row = idx / VPR;
            const int cv = idx % VPR;
            buf[u] = row < n ? *reinterpret_cast<const uint4*>(src + (size_t)row * stride + cv * VE)
                             : uint4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void commit(float* dst, int tid) const
    {
        static_assert(LD % 4 == 0, "16-byte LDS rows");
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int idx = tid + u * NT;
            float4* d = reinterpret_cast<float4*>(dst + (idx / VPR) * LD + (idx % VPR) * VE);
            if constexpr (sizeof(E) == 2) {
                const unsigned w[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
                d[0] = float4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                              __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
                d[1] = float4{__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                              __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u)};
            } else {
                d[0] = float4{__uint_as_float(buf[u].x), __uint_as_float(buf[u].y),
                              __uint_as_float(buf[u].z), __uint_as_float(buf[u].w)};
            }
        }
    }
};

template <int D, int LD, typename E>
__device__ __forceinline__ void stage(float* dst, const E* __restrict__ src, size_t stride, int n,
                                      int tid)
{
    Tile<E, D, LD> t;
    t.fetch(src, stride, n, tid);
    t.commit(dst, tid);
}

// sum over the 16 lanes of a lane group (lanes 16 g .. 16 g + 15)
__device__ __forceinline__ float sum16(float x)
{
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// Scans over the 64 lanes of a wavefront, lane i holding row i: the affine
// recurrence x_i = m_i x_{i-1} + c_i from x_{-1} = 0 (prefix), and
// y_i = c_i + m_i y_{i+1} from y_64 = 0 (suffix).  Six shuffle steps each.
__device__ __forceinline__ float prefix_affine(float m, float c, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float mp = __shfl_up(m, d);
        const float cp = __shfl_up(c, d);
        if (lane >= d) {
            c = m * cp + c;
            m = m * mp;
        }
    }
    return c;
}
__device__ __forceinline__ float suffix_affine(float m, float c, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float mn = __shfl_down(m, d);
        const float cn = __shfl_down(c, d);
        if (lane + d < 64) {
            c = c + m * cn;
            m = m * mn;
        }
    }
    return c;
}

// ---------------------------------------------------------------------------
// Reverse scan.  Wavefront w keeps 16 columns of dS and dM in fp32 MFMA
// accumulators (rows 16 rt + 4 lg + r, column wcol + l16), as the forward
// scan keeps S and M.
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
__global__ __launch_bounds__(NT) void bwd_scan_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ dO,
    const E* __restrict__ Tw, const E* __restrict__ Aw, const float* __restrict__ Vw,
    const float* dST, const float* dMT, E* __restrict__ Hd, float* __restrict__ dv,
    float* dS0, float* dM0, int T, int H, int NC)
{
    constexpr int TV = 64;
    constexpr int NTILE = DV / TV;
    constexpr int RT = DK / 16;
    constexpr int LDK = DK + 4;
    constexpr int LDV = TV + 4;
    constexpr int LDC = CH + 4;
    __shared__ __align__(16) float Qs[CH * LDK];
    __shared__ __align__(16) float Ks[CH * LDK];
    __shared__ __align__(16) float Gs[CH * LDV];   // dO, this workgroup's columns
    __shared__ __align__(16) float Ts[CH * LDC];
    __shared__ __align__(16) float As[CH * LDC];
    __shared__ __align__(16) float vecs[6 * CH];
    // bf16 I/O: every product below runs on 16x16x32 bf16 steps in the k
    // order of Mma<__bf16>::perm_row.  q, k, dO, T and A are exact in bf16;
    // the carried dS', dM' are rounded to bf16 in K dS', K dM' (the rounding
    // their copies in Hd get); the fp32 intermediates (dVt and the gate-scaled
    // rows of dO and dR) are split into a bf16 head and a bf16 remainder, two
    // steps each, about 16 bits.  All sums and the carried state gradients
    // stay fp32.
    constexpr bool BF = sizeof(E) == 2;
    using MB = Mma<__bf16>;
    auto split8 = [](const float* x, bf16x8& hd, bf16x8& rs) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            hd[j] = static_cast<__bf16>(x[j]);
            rs[j] = static_cast<__bf16>(x[j] - static_cast<float>(hd[j]));
        }
    };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int tile = (int)(blockIdx.x % NTILE);
    const int bh = (int)(blockIdx.x / NTILE);
    const int h = bh % H;
    const int b = bh / H;
    const int lcol = 16 * wave + l16;        // column inside the workgroup's 64
    const int wcol = tile * TV + 16 * wave;  // first column of this wavefront

    f32x4 Sa[RT], Ma[RT];
    const size_t sbase = (size_t)bh * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const size_t x = sbase + (size_t)(16 * rt + 4 * lg + r) * DV + wcol + l16;
            Sa[rt][r] = dST ? dST[x] : 0.f;
            Ma[rt][r] = dMT ? dMT[x] : 0.f;
        }

    Tile<E, DK, LDK> pq, pk;
    Tile<E, TV, LDV> pg;
    Tile<E, CH, LDC> pt, pa;
    float pvec[2];
    auto fetch = [&](int c) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const size_t tok0 = ((size_t)b * T + t0) * H + h;
        const size_t chn = (size_t)bh * NC + c;
        pq.fetch(q + tok0 * DK, (size_t)H * DK, n, tid);
        pk.fetch(k + tok0 * DK, (size_t)H * DK, n, tid);
        pg.fetch(dO + tok0 * DV + tile * TV, (size_t)H * DV, n, tid);
        pt.fetch(Tw + chn * CH * CH, CH, CH, tid);
        pa.fetch(Aw + chn * CH * CH, CH, CH, tid);
#pragma unroll
        for (int u = 0; u < 2; ++u)
            pvec[u] = tid + u * NT < 6 * CH ? Vw[chn * NVEC * CH + tid + u * NT] : 0.f;
    };
    fetch(NC - 1);

    for (int c = NC - 1; c >= 0; --c) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const size_t tok0 = ((size_t)b * T + t0) * H + h;
        const size_t chn = (size_t)bh * NC + c;

        __syncthreads();
        pq.commit(Qs, tid);
        pk.commit(Ks, tid);
        pg.commit(Gs, tid);
        pt.commit(Ts, tid);
        pa.commit(As, tid);
#pragma unroll
        for (int u = 0; u < 2; ++u)
            if (tid + u * NT < 6 * CH) vecs[tid + u * NT] = pvec[u];
        __syncthreads();
        if (c > 0) fetch(c - 1);

        // the exit-state gradients of this chunk, for bwd_grad_kernel
        {
            E* hd = Hd + chn * 2 * DK * DV;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const size_t x = (size_t)(16 * rt + 4 * lg + r) * DV + wcol + l16;
                    hd[x] = to_elem<E>(Sa[rt][r]);
                    hd[(size_t)DK * DV + x] = to_elem<E>(Ma[rt][r]);
                }
        }

        // K dS', K dM' (rows i, this wavefront's columns)
        f32x4 xs[4], xm[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) xs[ct] = xm[ct] = zero4();
        if constexpr (BF) {
            // (dS' and dM' get the rounding their copies in Hd get)
#pragma unroll
            for (int s2 = 0; s2 < DK / 32; ++s2) {
                const bf16x8 bS = Mma<__bf16>::from_acc(Sa, s2);
                const bf16x8 bM = Mma<__bf16>::from_acc(Ma, s2);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const float* kp = Ks + (16 * ct + l16) * LDK + 32 * s2 + 4 * lg;
                    const float4 u = *reinterpret_cast<const float4*>(kp);
                    const float4 w = *reinterpret_cast<const float4*>(kp + 16);
                    const bf16x8 aK = {(__bf16)u.x, (__bf16)u.y, (__bf16)u.z, (__bf16)u.w,
                                       (__bf16)w.x, (__bf16)w.y, (__bf16)w.z, (__bf16)w.w};
                    xs[ct] = Mma<__bf16>::mma(aK, bS, xs[ct]);
                    xm[ct] = Mma<__bf16>::mma(aK, bM, xm[ct]);
                }
            }
        } else
#pragma unroll
        for (int sb = 0; sb < DK / 16; ++sb) {
            float4 a4[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                a4[ct] = *reinterpret_cast<const float4*>(Ks + (16 * ct + l16) * LDK + 16 * sb + 4 * lg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // k = perm_row(4 sb + e, lg) = 16 sb + 4 lg + e
                const float bS = Sa[sb][e];
                const float bM = Ma[sb][e];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const float aK = e == 0 ? a4[ct].x : e == 1 ? a4[ct].y : e == 2 ? a4[ct].z : a4[ct].w;
                    xs[ct] = MF::mma(aK, bS, xs[ct]);
                    xm[ct] = MF::mma(aK, bM, xm[ct]);
                }
            }
        }

        // dVt = A^T dO + Diag(ws) K dS' - Diag(wm) K dM'
        f32x4 dVt[4];
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * lg + r;
                dVt[it][r] = vecs[V_WS * CH + i] * xs[it][r] - vecs[V_WM * CH + i] * xm[it][r];
            }
        if constexpr (BF) {
#pragma unroll
            for (int s2 = 0; s2 < CH / 32; ++s2) {
                bf16x8 bO;
#pragma unroll
                for (int j = 0; j < 8; ++j) bO[j] = (__bf16)Gs[MB::perm_row(s2, lg, j) * LDV + lcol];
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    bf16x8 aA;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        aA[j] = (__bf16)As[MB::perm_row(s2, lg, j) * LDC + 16 * it + l16];
                    dVt[it] = MB::mma(aA, bO, dVt[it]);
                }
            }
        } else
#pragma unroll
        for (int s = 0; s < CH / 4; ++s) {
            const int kr = MF::perm_row(s, lg, 0);
            const float bO = Gs[kr * LDV + lcol];
#pragma unroll
            for (int it = 0; it < 4; ++it)
                dVt[it] = MF::mma(As[kr * LDC + 16 * it + l16], bO, dVt[it]);
        }

        // dR = T^T dVt, written as dv
        f32x4 dR[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) dR[it] = zero4();
        if constexpr (BF) {
#pragma unroll
            for (int s2 = 0; s2 < CH / 32; ++s2) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[j] = dVt[2 * s2][j];
                    x[4 + j] = dVt[2 * s2 + 1][j];
                }
                bf16x8 vh, vr;
                split8(x, vh, vr);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    bf16x8 aT;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        aT[j] = (__bf16)Ts[MB::perm_row(s2, lg, j) * LDC + 16 * it + l16];
                    dR[it] = MB::mma(aT, vh, dR[it]);
                    dR[it] = MB::mma(aT, vr, dR[it]);
                }
            }
        } else
#pragma unroll
        for (int s = 0; s < CH / 4; ++s) {
            const float bV = MF::from_acc(dVt, s);
            const int kr = MF::perm_row(s, lg, 0);
#pragma unroll
            for (int it = 0; it < 4; ++it)
                dR[it] = MF::mma(Ts[kr * LDC + 16 * it + l16], bV, dR[it]);
        }
        {
            float* dvb = dv + tok0 * DV + wcol + l16;
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * it + 4 * lg + r;
                    if (i < n) dvb[(size_t)i * H * DV] = dR[it][r];
                }
        }

        // carry back: dS <- abar_n dS' + Q^T Diag(abar) dO - K^T Diag(abar) dR,
        //             dM <- mubar_n dM' - b_n dS' - Q^T Diag(b) dO + K^T Diag(ab1) dR
        const float abn = vecs[V_SCAL * CH + 0];
        const float bn = vecs[V_SCAL * CH + 1];
        const float mbn = vecs[V_SCAL * CH + 2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4 so = Sa[rt];
            Sa[rt] = abn * so;
            Ma[rt] = mbn * Ma[rt] - bn * so;
        }
        if constexpr (BF) {
#pragma unroll
            for (int s2 = 0; s2 < CH / 32; ++s2) {
                float xs8[8], xm8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int kr = MB::perm_row(s2, lg, j);
                    const float g = Gs[kr * LDV + lcol];
                    xs8[j] = vecs[V_ABAR * CH + kr] * g;
                    xm8[j] = -vecs[V_B * CH + kr] * g;
                }
                bf16x8 sh, sr, mh, mr;
                split8(xs8, sh, sr);
                split8(xm8, mh, mr);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    bf16x8 aQ;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        aQ[j] = (__bf16)Qs[MB::perm_row(s2, lg, j) * LDK + 16 * rt + l16];
                    Sa[rt] = MB::mma(aQ, sh, Sa[rt]);
                    Sa[rt] = MB::mma(aQ, sr, Sa[rt]);
                    Ma[rt] = MB::mma(aQ, mh, Ma[rt]);
                    Ma[rt] = MB::mma(aQ, mr, Ma[rt]);
                }
            }
#pragma unroll
            for (int s2 = 0; s2 < CH / 32; ++s2) {
                float xs8[8], xm8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int kr = MB::perm_row(s2, lg, j);
                    const float r = j < 4 ? dR[2 * s2][j] : dR[2 * s2 + 1][j - 4];
                    xs8[j] = -vecs[V_ABAR * CH + kr] * r;
                    xm8[j] = vecs[V_AB1 * CH + kr] * r;
                }
                bf16x8 sh, sr, mh, mr;
                split8(xs8, sh, sr);
                split8(xm8, mh, mr);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    bf16x8 aK;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        aK[j] = (__bf16)Ks[MB::perm_row(s2, lg, j) * LDK + 16 * rt + l16];
                    Sa[rt] = MB::mma(aK, sh, Sa[rt]);
                    Sa[rt] = MB::mma(aK, sr, Sa[rt]);
                    Ma[rt] = MB::mma(aK, mh, Ma[rt]);
                    Ma[rt] = MB::mma(aK, mr, Ma[rt]);
                }
            }
        } else {
#pragma unroll
        for (int s = 0; s < CH / 4; ++s) {
            const int kr = MF::perm_row(s, lg, 0);
            const float g = Gs[kr * LDV + lcol];
            const float bS = vecs[V_ABAR * CH + kr] * g;
            const float bM = -vecs[V_B * CH + kr] * g;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const float aQ = Qs[kr * LDK + 16 * rt + l16];
                Sa[rt] = MF::mma(aQ, bS, Sa[rt]);
                Ma[rt] = MF::mma(aQ, bM, Ma[rt]);
            }
        }
#pragma unroll
        for (int s = 0; s < CH / 4; ++s) {
            const float bS = MF::from_acc_scaled(dR, s, lg, vecs + V_ABAR * CH, -1.f);
            const float bM = MF::from_acc_scaled(dR, s, lg, vecs + V_AB1 * CH, 1.f);
            const int kr = MF::perm_row(s, lg, 0);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const float aK = Ks[kr * LDK + 16 * rt + l16];
                Sa[rt] = MF::mma(aK, bS, Sa[rt]);
                Ma[rt] = MF::mma(aK, bM, Ma[rt]);
            }
        }
        }
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const size_t x = sbase + (size_t)(16 * rt + 4 * lg + r) * DV + wcol + l16;
            if (dS0) dS0[x] = Sa[rt][r];
            if (dM0) dM0[x] = Ma[rt][r];
        }
}

// ---------------------------------------------------------------------------
// Forward re-scan: the chunk-entry states and Vt of every chunk.
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV, bool SAVED>
__global__ __launch_bounds__(NT) void bwd_rescan_kernel(
    const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ Tw,
    const float* __restrict__ Vw, const float* S0, const float* M0, E* __restrict__ Hs,
    float* __restrict__ Vts, int T, int H, int NC)
{
    // SAVED: v holds the forward's residuals Vt ([B, T, H, DV]); the chunk's
    // Vt is then read instead of solved for, and only the states are rebuilt
    constexpr int TV = 64;
    constexpr int NTILE = DV / TV;
    constexpr int RT = DK / 16;
    constexpr int LDK = DK + 4;
    constexpr int LDV = TV + 4;
    constexpr int LDC = CH + 4;
    __shared__ __align__(16) float Ks[CH * LDK];
    __shared__ __align__(16) float Vs[CH * LDV];
    __shared__ __align__(16) float Ts[CH * LDC];
    __shared__ float vecs[6 * CH];
    // bf16 I/O: the products run on 16x16x32 bf16 steps in the k order of
    // Mma<__bf16>::perm_row with fp32 sums.  k and T are exact in bf16; S and M
    // are rounded to bf16 in K S, K M, as in the forward; R and the
    // weight-scaled rows of Vt are split into a bf16 head and a bf16
    // remainder, two steps each, about 16 bits.  The carried states stay fp32.
    constexpr bool BF = sizeof(E) == 2;
    using MB = Mma<__bf16>;
    auto split8 = [](const float* x, bf16x8& hd, bf16x8& rs) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            hd[j] = static_cast<__bf16>(x[j]);
            rs[j] = static_cast<__bf16>(x[j] - static_cast<float>(hd[j]));
        }
    };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int tile = (int)(blockIdx.x % NTILE);
    const int bh = (int)(blockIdx.x / NTILE);
    const int h = bh % H;
    const int b = bh / H;
    const int lcol = 16 * wave + l16;
    const int wcol = tile * TV + 16 * wave;

    f32x4 Sa[RT], Ma[RT];
    const size_t sbase = (size_t)bh * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const size_t x = sbase + (size_t)(16 * rt + 4 * lg + r) * DV + wcol + l16;
            Sa[rt][r] = S0 ? S0[x] : 0.f;
            Ma[rt][r] = M0 ? M0[x] : 0.f;
        }

    Tile<E, DK, LDK> pk;
    Tile<E, TV, LDV> pv;
    Tile<E, CH, LDC> pt;
    float pvec[2];
    auto fetch = [&](int c) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const size_t tok0 = ((size_t)b * T + t0) * H + h;
        const size_t chn = (size_t)bh * NC + c;
        pk.fetch(k + tok0 * DK, (size_t)H * DK, n, tid);
        pv.fetch(v + tok0 * DV + tile * TV, (size_t)H * DV, n, tid);
        if (!SAVED) pt.fetch(Tw + chn * CH * CH, CH, CH, tid);
#pragma unroll
        for (int u = 0; u < 2; ++u)
            pvec[u] = tid + u * NT < 6 * CH ? Vw[chn * NVEC * CH + tid + u * NT] : 0.f;
    };
    fetch(0);

    for (int c = 0; c < NC; ++c) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const size_t tok0 = ((size_t)b * T + t0) * H + h;
        const size_t chn = (size_t)bh * NC + c;
        (void)tok0;

        __syncthreads();
        pk.commit(Ks, tid);
        pv.commit(Vs, tid);
        if (!SAVED) pt.commit(Ts, tid);
#pragma unroll
        for (int u = 0; u < 2; ++u)
            if (tid + u * NT < 6 * CH) vecs[tid + u * NT] = pvec[u];
        __syncthreads();
        if (c + 1 < NC) fetch(c + 1);

        {
            E* hs = Hs + chn * 2 * DK * DV;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const size_t x = (size_t)(16 * rt + 4 * lg + r) * DV + wcol + l16;
                    hs[x] = to_elem<E>(Sa[rt][r]);
                    hs[(size_t)DK * DV + x] = to_elem<E>(Ma[rt][r]);
                }
        }

        f32x4 Vt[4];
        if constexpr (!SAVED) {
        f32x4 xs[4], xm[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) xs[ct] = xm[ct] = zero4();
        if constexpr (BF) {
#pragma unroll
            for (int s2 = 0; s2 < DK / 32; ++s2) {
                const bf16x8 bS = MB::from_acc(Sa, s2);
                const bf16x8 bM = MB::from_acc(Ma, s2);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const float* kp = Ks + (16 * ct + l16) * LDK + 32 * s2 + 4 * lg;
                    const float4 u = *reinterpret_cast<const float4*>(kp);
                    const float4 w = *reinterpret_cast<const float4*>(kp + 16);
                    const bf16x8 aK = {(__bf16)u.x, (__bf16)u.y, (__bf16)u.z, (__bf16)u.w,
                                       (__bf16)w.x, (__bf16)w.y, (__bf16)w.z, (__bf16)w.w};
                    xs[ct] = MB::mma(aK, bS, xs[ct]);
                    xm[ct] = MB::mma(aK, bM, xm[ct]);
                }
            }
        } else
#pragma unroll
        for (int sb = 0; sb < DK / 16; ++sb) {
            float4 a4[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                a4[ct] = *reinterpret_cast<const float4*>(Ks + (16 * ct + l16) * LDK + 16 * sb + 4 * lg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // k = perm_row(4 sb + e, lg) = 16 sb + 4 lg + e
                const float bS = Sa[sb][e];
                const float bM = Ma[sb][e];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const float aK = e == 0 ? a4[ct].x : e == 1 ? a4[ct].y : e == 2 ? a4[ct].z : a4[ct].w;
                    xs[ct] = MF::mma(aK, bS, xs[ct]);
                    xm[ct] = MF::mma(aK, bM, xm[ct]);
                }
            }
        }
        f32x4 R[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ct + 4 * lg + r;
                R[ct][r] = Vs[i * LDV + lcol] - vecs[V_ABAR * CH + i] * xs[ct][r] +
                           vecs[V_AB1 * CH + i] * xm[ct][r];
            }
#pragma unroll
        for (int it = 0; it < 4; ++it) Vt[it] = zero4();
        if constexpr (BF) {
#pragma unroll
            for (int s2 = 0; s2 < CH / 32; ++s2) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[j] = R[2 * s2][j];
                    x[4 + j] = R[2 * s2 + 1][j];
                }
                bf16x8 rh, rr;
                split8(x, rh, rr);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const float* tp = Ts + (16 * it + l16) * LDC + 32 * s2 + 4 * lg;
                    const float4 u = *reinterpret_cast<const float4*>(tp);
                    const float4 w = *reinterpret_cast<const float4*>(tp + 16);
                    const bf16x8 aT = {(__bf16)u.x, (__bf16)u.y, (__bf16)u.z, (__bf16)u.w,
                                       (__bf16)w.x, (__bf16)w.y, (__bf16)w.z, (__bf16)w.w};
                    Vt[it] = MB::mma(aT, rh, Vt[it]);
                    Vt[it] = MB::mma(aT, rr, Vt[it]);
                }
            }
        } else
#pragma unroll
        for (int sb = 0; sb < CH / 16; ++sb) {
            float4 t4[4];
#pragma unroll
            for (int it = 0; it < 4; ++it)
                t4[it] = *reinterpret_cast<const float4*>(Ts + (16 * it + l16) * LDC + 16 * sb + 4 * lg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float bR = R[sb][e];
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const float aT = e == 0 ? t4[it].x : e == 1 ? t4[it].y : e == 2 ? t4[it].z : t4[it].w;
                    Vt[it] = MF::mma(aT, bR, Vt[it]);
                }
            }
        }
        {
            float* vb = Vts + chn * CH * DV + wcol + l16;
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int r = 0; r < 4; ++r) vb[(size_t)(16 * it + 4 * lg + r) * DV] = Vt[it][r];
        }

        }
        const float abn = vecs[V_SCAL * CH + 0];
        const float bn = vecs[V_SCAL * CH + 1];
        const float mbn = vecs[V_SCAL * CH + 2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            Sa[rt] = abn * Sa[rt] - bn * Ma[rt];
            Ma[rt] = mbn * Ma[rt];
        }
        if constexpr (BF) {
#pragma unroll
            for (int s2 = 0; s2 < CH / 32; ++s2) {
                float xs8[8], xm8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int kr = MB::perm_row(s2, lg, j);
                    float vt;
                    if constexpr (SAVED) vt = Vs[kr * LDV + lcol];
                    else vt = j < 4 ? Vt[2 * s2][j] : Vt[2 * s2 + 1][j - 4];
                    xs8[j] = vecs[V_WS * CH + kr] * vt;
                    xm8[j] = -(vecs[V_WM * CH + kr] * vt);
                }
                bf16x8 sh, sr, mh, mr;
                split8(xs8, sh, sr);
                split8(xm8, mh, mr);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    bf16x8 aK;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        aK[j] = (__bf16)Ks[MB::perm_row(s2, lg, j) * LDK + 16 * rt + l16];
                    Sa[rt] = MB::mma(aK, sh, Sa[rt]);
                    Sa[rt] = MB::mma(aK, sr, Sa[rt]);
                    Ma[rt] = MB::mma(aK, mh, Ma[rt]);
                    Ma[rt] = MB::mma(aK, mr, Ma[rt]);
                }
            }
        } else
#pragma unroll
        for (int s = 0; s < CH / 4; ++s) {
            const int kr = MF::perm_row(s, lg, 0);
            float bS, bM;
            if constexpr (SAVED) {
                const float vt = Vs[kr * LDV + lcol];
                bS = vecs[V_WS * CH + kr] * vt;
                bM = -(vecs[V_WM * CH + kr] * vt);
            } else {
                bS = MF::from_acc_scaled(Vt, s, lg, vecs + V_WS * CH, 1.f);
                bM = MF::from_acc_scaled(Vt, s, lg, vecs + V_WM * CH, -1.f);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const float aK = Ks[kr * LDK + 16 * rt + l16];
                Sa[rt] = MF::mma(aK, bS, Sa[rt]);
                Ma[rt] = MF::mma(aK, bM, Ma[rt]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Per-chunk gradients: one workgroup per (b, h, chunk), all columns.
//
// C x DK results (dq, dk and the state products) are split over the four
// wavefronts by column tiles: wavefront w owns d-tiles w * DT .. w * DT + DT - 1
// (DT = DK / 64) and all four row tiles.  C x C results: wavefront w owns row
// tile w and all four column tiles.
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct GradSmem {
    static constexpr int LDK = DK + 4;
    static constexpr int LDV = DV + 4;
    static constexpr int LD = LDK > LDV ? LDK : LDV;
    static constexpr int SLOT = CH * LD;     // floats of one C x D tile
    static constexpr int LDC = CH + 4;
    static constexpr int CM = CH * LDC;      // floats of one C x C matrix
    static constexpr int NV = 24;            // vectors of CH floats
    static constexpr int FLOATS = 3 * SLOT + 3 * CM + NV * CH + 8;
};

// vector rows of GradSmem
constexpr int G_A = 0, G_M = 1, G_E = 2, G_S = 3;          // gates alpha, mu, eta, beta
constexpr int G_AB = 4, G_MB = 5, G_B = 6;                   // abar, mubar, b
constexpr int G_RX1 = 7, G_RX2 = 8, G_RY1 = 9, G_RY2 = 10;   // row dots
constexpr int G_RZ1 = 11, G_RZ2 = 12, G_RKH = 13, G_RP = 14;
constexpr int G_DA = 15, G_DM = 16, G_DE = 17, G_DS = 18;    // gate gradients
constexpr int G_DAB = 19, G_DMB = 20, G_DB = 21;             // coefficient gradients
constexpr int G_RED = 22;                                    // 2 rows: reduction scratch

template <typename E, int DK, int DV>
__global__ __launch_bounds__(NT) void bwd_grad_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ dO,
    const float* __restrict__ dv, const float* __restrict__ Vts, const E* __restrict__ Vsaved,
    const E* __restrict__ Hs,
    const E* __restrict__ Hd, const float* __restrict__ alpha, const float* __restrict__ mu,
    const float* __restrict__ eta, const float* __restrict__ beta, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dalpha, float* __restrict__ dmu,
    float* __restrict__ deta, float* __restrict__ dbeta, int T, int H, int NC)
{
    using SM = GradSmem<DK, DV>;
    constexpr int LD = SM::LD;
    constexpr int LDC = SM::LDC;
    constexpr int DT = DK / 64;   // d-tiles per wavefront
    __shared__ __align__(16) float smem[SM::FLOATS];
    float* slot0 = smem;
    float* slot1 = smem + SM::SLOT;
    float* slot2 = smem + 2 * SM::SLOT;
    float* Gm = smem + 3 * SM::SLOT;     // Gamma
    float* Cm1 = Gm + SM::CM;
    float* Cm2 = Cm1 + SM::CM;
    float* vec = Cm2 + SM::CM;
    float* scal = vec + SM::NV * CH;     // 3 state inner products

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int c = (int)(blockIdx.x % NC);
    const int bh = (int)(blockIdx.x / NC);
    const int h = bh % H;
    const int b = bh / H;
    const int t0 = c * CH;
    const int n = min(CH, T - t0);
    const size_t tok0 = ((size_t)b * T + t0) * H + h;
    const size_t chn = (size_t)bh * NC + c;
    // the chunk's states, stored in the I/O type (bf16 states are the rounding
    // the forward's MFMA operands make too)
    const E* S0 = Hs + chn * 2 * DK * DV;
    const E* M0 = S0 + DK * DV;
    const E* dS = Hd + chn * 2 * DK * DV;
    const E* dM = dS + DK * DV;
    constexpr int SV = 16 / sizeof(E);   // state values per 16-byte load
    auto unpack = [](const uint4& w, float* f) {
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
    };
    auto V = [&](int row) { return vec + row * CH; };

    // ---- gates, coefficient vectors, Gamma ----------------------------------
    for (int i = tid; i < CH; i += NT) {
        const bool in = i < n;
        const size_t g = tok0 + (size_t)i * H;
        V(G_A)[i] = in ? alpha[g] : 1.f;
        V(G_M)[i] = in && mu ? mu[g] : 0.f;
        V(G_E)[i] = in ? eta[g] : 0.f;
        V(G_S)[i] = in ? (beta ? beta[g] : 1.f) : 0.f;
    }
    for (int i = tid; i < (SM::NV - G_RX1) * CH; i += NT) vec[G_RX1 * CH + i] = 0.f;
    __syncthreads();
    if (wave == 0) {
        // abar, mubar (prefix products) and b_i = alpha_i b_{i-1} + beta_i mubar_i
        const float a = V(G_A)[lane], m = V(G_M)[lane];
        float pa = a, pm = m;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float ua = __shfl_up(pa, d), um = __shfl_up(pm, d);
            if (lane >= d) {
                pa *= ua;
                pm *= um;
            }
        }
        V(G_AB)[lane] = pa;
        V(G_MB)[lane] = pm;
        V(G_B)[lane] = prefix_affine(a, V(G_S)[lane] * pm, lane);
    }
    // Gamma by columns (thread j < CH): rows < j are zero; m lives in Cm1 for now
    if (tid < CH) {
        const int j = tid;
        float g = 0.f, m = 1.f;
        for (int i = 0; i < CH; ++i) {
            if (i == j) {
                g = V(G_S)[j];
                m = 1.f;
            } else if (i > j) {
                m = V(G_M)[i] * m;
                g = V(G_A)[i] * g + V(G_S)[i] * m;
            }
            Gm[i * LDC + j] = i >= j ? g : 0.f;
            Cm1[i * LDC + j] = i >= j ? m : 0.f;
        }
    }
    __syncthreads();
    // last-row weights ws_j = eta_j gamma_{n-1,j}, wm_j = eta_j m_{n-1,j}
    // (kept in the reduction rows until the state products are done)
    float* ws = V(G_RED);
    float* wm = V(G_RED + 1);
    for (int j = tid; j < CH; j += NT) {
        ws[j] = V(G_E)[j] * Gm[(n - 1) * LDC + j];
        wm[j] = V(G_E)[j] * Cm1[(n - 1) * LDC + j];
    }
    // the three state inner products (each thread a strided share, then a
    // fixed-order reduction over the four wavefronts)
    {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f;
        constexpr int NF = DK * DV / SV / NT;   // 16-byte loads per thread and array
        constexpr int BATCH = NF < 4 ? NF : 4;
        for (int u0 = 0; u0 < NF; u0 += BATCH) {
            uint4 s0[BATCH], m0[BATCH], ds[BATCH], dm[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int x = SV * (tid + (u0 + u) * NT);
                s0[u] = *reinterpret_cast<const uint4*>(S0 + x);
                m0[u] = *reinterpret_cast<const uint4*>(M0 + x);
                ds[u] = *reinterpret_cast<const uint4*>(dS + x);
                dm[u] = *reinterpret_cast<const uint4*>(dM + x);
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                float fs[SV], fm[SV], fd[SV], fe[SV];
                unpack(s0[u], fs);
                unpack(m0[u], fm);
                unpack(ds[u], fd);
                unpack(dm[u], fe);
#pragma unroll
                for (int e = 0; e < SV; ++e) {
                    a0 += fd[e] * fs[e];
                    a1 += fd[e] * fm[e];
                    a2 += fe[e] * fm[e];
                }
            }
        }
        for (int o = 32; o >= 1; o >>= 1) {
            a0 += __shfl_xor(a0, o);
            a1 += __shfl_xor(a1, o);
            a2 += __shfl_xor(a2, o);
        }
        __shared__ float part[3][4];
        if (lane == 0) {
            part[0][wave] = a0;
            part[1][wave] = a1;
            part[2][wave] = a2;
        }
        __syncthreads();
        if (tid < 3) scal[tid] = (part[tid][0] + part[tid][1]) + (part[tid][2] + part[tid][3]);
    }

    // ---- state products ------------------------------------------------------
    // For a C x DV row operand X in LDS and a DK x DV state St in HBM, the
    // product X St^T (C x DK): this wavefront's tiles, k over the DV columns
    // in the fp32 k-permuted order, 4 state values per 16-byte load.
    auto state_product = [&](const float* X, const E* St, f32x4 (*acc)[DT]) {
        // k order: block kb of KB = 4 SV columns, lane group lg takes columns
        // KB kb + SV lg + e (e < SV) from one 16-byte load of the state row
        constexpr int KB = 4 * SV;
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[it][dt] = zero4();
        // this wavefront's rows of the state, all DV columns, loaded at once
        uint4 sva[DV / KB][DT];
#pragma unroll
        for (int kb = 0; kb < DV / KB; ++kb)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = 16 * (wave * DT + dt) + l16;
                sva[kb][dt] =
                    *reinterpret_cast<const uint4*>(St + (size_t)d * DV + KB * kb + SV * lg);
            }
        if constexpr (sizeof(E) == 2) {
            // bf16 states: one 16x16x32 bf16 step per block of 32 columns.  The
            // lane's 16-byte load of a state row is its B fragment as it stands
            // (k = 32 kb + 8 lg + j); the A fragment is the same 8 columns of
            // X's row, rounded to bf16 (exact for dO and for saved Vt).
#pragma unroll
            for (int kb = 0; kb < DV / KB; ++kb) {
                bf16x8 bv[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) bv[dt] = __builtin_bit_cast(bf16x8, sva[kb][dt]);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const float* xr = X + (16 * it + l16) * LD + KB * kb + SV * lg;
                    const float4 x0 = *reinterpret_cast<const float4*>(xr);
                    const float4 x1 = *reinterpret_cast<const float4*>(xr + 4);
                    const bf16x8 a = {(__bf16)x0.x, (__bf16)x0.y, (__bf16)x0.z, (__bf16)x0.w,
                                      (__bf16)x1.x, (__bf16)x1.y, (__bf16)x1.z, (__bf16)x1.w};
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
                        acc[it][dt] = Mma<__bf16>::mma(a, bv[dt], acc[it][dt]);
                }
            }
            return;
        }
#pragma unroll
        for (int kb = 0; kb < DV / KB; ++kb) {
            float sv[DT][SV];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) unpack(sva[kb][dt], sv[dt]);
#pragma unroll
            for (int h4 = 0; h4 < SV / 4; ++h4) {
                float4 xa[4];
#pragma unroll
                for (int it = 0; it < 4; ++it)
                    xa[it] = *reinterpret_cast<const float4*>(
                        X + (16 * it + l16) * LD + KB * kb + SV * lg + 4 * h4);
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
                    for (int it = 0; it < 4; ++it) {
                        const float a = e4 == 0 ? xa[it].x : e4 == 1 ? xa[it].y
                                      : e4 == 2 ? xa[it].z : xa[it].w;
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt)
                            acc[it][dt] = MF::mma(a, sv[dt][4 * h4 + e4], acc[it][dt]);
                    }
            }
        }
    };
    // row dot of a C x DK accumulator set with a C x DK LDS operand Y: adds
    // this wavefront's share into red[wave][i]; the caller sums the four
    float* red = Cm2;   // [4][CH] scratch (Cm2 is free until the C x C phase)
    auto row_dot = [&](const f32x4 (*acc)[DT], const float* Y, float* out_row) {
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * lg + r;
                float p = 0.f;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    p += acc[it][dt][r] * Y[i * LD + 16 * (wave * DT + dt) + l16];
                p = sum16(p);
                if (l16 == 0) red[wave * CH + i] = p;
            }
        __syncthreads();
        for (int i = tid; i < CH; i += NT)
            out_row[i] = (red[i] + red[CH + i]) + (red[2 * CH + i] + red[3 * CH + i]);
        __syncthreads();
    };

    // this wavefront's row tile of X Y^T (C x C), k over KD columns of both,
    // 16-byte k-permuted reads
    auto cc_product = [&](const float* X, const float* Y, int KD, float sign, f32x4* acc) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[jt] = zero4();
        for (int kb = 0; kb < KD / 16; ++kb) {
            const float4 a4 =
                *reinterpret_cast<const float4*>(X + (16 * wave + l16) * LD + 16 * kb + 4 * lg);
            float4 b4[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                b4[jt] = *reinterpret_cast<const float4*>(Y + (16 * jt + l16) * LD + 16 * kb + 4 * lg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = sign * (e == 0 ? a4.x : e == 1 ? a4.y : e == 2 ? a4.z : a4.w);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    const float bv = e == 0 ? b4[jt].x : e == 1 ? b4[jt].y : e == 2 ? b4[jt].z : b4[jt].w;
                    acc[jt] = MF::mma(a, bv, acc[jt]);
                }
            }
        }
    };

    // the same on bf16 MFMA, for operands that hold bf16 values (inputs in the
    // I/O type and saved Vt): one 16x16x32 step per 32 columns, lane group lg
    // taking columns 32 kb + 8 lg .. 32 kb + 8 lg + 7 of both rows
    auto cc_product_bf16 = [&](const float* X, const float* Y, int KD, f32x4* acc) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) acc[jt] = zero4();
        auto frag = [](const float* p) {
            const float4 u = *reinterpret_cast<const float4*>(p);
            const float4 w = *reinterpret_cast<const float4*>(p + 4);
            return bf16x8{(__bf16)u.x, (__bf16)u.y, (__bf16)u.z, (__bf16)u.w,
                          (__bf16)w.x, (__bf16)w.y, (__bf16)w.z, (__bf16)w.w};
        };
        for (int kb = 0; kb < KD / 32; ++kb) {
            const bf16x8 a = frag(X + (16 * wave + l16) * LD + 32 * kb + 8 * lg);
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                acc[jt] = Mma<__bf16>::mma(a, frag(Y + (16 * jt + l16) * LD + 32 * kb + 8 * lg),
                                           acc[jt]);
        }
    };
    constexpr bool BF = sizeof(E) == 2;

    f32x4 dQa[4][DT], dKa[4][DT], P1[4][DT], P2[4][DT];
    f32x4 cA[4], cL[4], cK[4];   // C x C tiles: dA, dL, K K^T (row tile = wave)

    // phase 1: slot0 = Vt, slot1 = dO, slot2 = Q.  The three fetches are in
    // flight together for bf16 inputs; fp32 inputs stage one tile at a time
    // (three fp32 tiles in registers at once overflow the register file).
    __syncthreads();
    if constexpr (sizeof(E) == 2) {
        Tile<float, DV, LD> t0_;
        Tile<E, DV, LD> t1_;
        Tile<E, DK, LD> t2_;
        if (!Vsaved) t0_.fetch(Vts + chn * CH * DV, DV, n, tid);
        t1_.fetch(dO + tok0 * DV, (size_t)H * DV, n, tid);
        t2_.fetch(q + tok0 * DK, (size_t)H * DK, n, tid);
        if (Vsaved) stage<DV, LD>(slot0, Vsaved + tok0 * DV, (size_t)H * DV, n, tid);
        else t0_.commit(slot0, tid);
        t1_.commit(slot1, tid);
        t2_.commit(slot2, tid);
    } else {
        if (Vsaved) stage<DV, LD>(slot0, Vsaved + tok0 * DV, (size_t)H * DV, n, tid);
        else stage<DV, LD>(slot0, Vts + chn * CH * DV, DV, n, tid);
        stage<DV, LD>(slot1, dO + tok0 * DV, (size_t)H * DV, n, tid);
        stage<DK, LD>(slot2, q + tok0 * DK, (size_t)H * DK, n, tid);
    }
    __syncthreads();
    // dA = dO Vt^T (lower triangle with the diagonal kept below)
    // (Vt recomputed in fp32 is rounded here, as in its state products)
    if constexpr (BF) cc_product_bf16(slot1, slot0, DV, cA);
    else cc_product(slot1, slot0, DV, 1.f, cA);
    state_product(slot1, S0, P1);   // dO S0^T
    state_product(slot1, M0, P2);   // dO M0^T
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * lg + r;
                dQa[it][dt][r] = V(G_AB)[i] * P1[it][dt][r] - V(G_B)[i] * P2[it][dt][r];
            }
    row_dot(P1, slot2, V(G_RX1));
    row_dot(P2, slot2, V(G_RX2));

    // phase 2: slot1 = dR, slot2 = K (Vt stays in slot0)
    if constexpr (sizeof(E) == 2) {
        Tile<float, DV, LD> t1_;
        Tile<E, DK, LD> t2_;
        t1_.fetch(dv + tok0 * DV, (size_t)H * DV, n, tid);
        t2_.fetch(k + tok0 * DK, (size_t)H * DK, n, tid);
        t1_.commit(slot1, tid);
        t2_.commit(slot2, tid);
    } else {
        stage<DV, LD>(slot1, dv + tok0 * DV, (size_t)H * DV, n, tid);
        stage<DK, LD>(slot2, k + tok0 * DK, (size_t)H * DK, n, tid);
    }
    __syncthreads();
    cc_product(slot1, slot0, DV, -1.f, cL);
    if constexpr (BF) cc_product_bf16(slot2, slot2, DK, cK);
    else cc_product(slot2, slot2, DK, 1.f, cK);
    state_product(slot1, S0, P1);   // dR S0^T
    state_product(slot1, M0, P2);   // dR M0^T
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * lg + r;
                const float ab1 = i > 0 ? V(G_A)[i] * V(G_B)[i - 1] : 0.f;
                dKa[it][dt][r] = -V(G_AB)[i] * P1[it][dt][r] + ab1 * P2[it][dt][r];
            }
    row_dot(P1, slot2, V(G_RY1));
    row_dot(P2, slot2, V(G_RY2));
    state_product(slot0, dS, P1);   // Vt dS'^T
    state_product(slot0, dM, P2);   // Vt dM'^T
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * lg + r;
                dKa[it][dt][r] += ws[i] * P1[it][dt][r] - wm[i] * P2[it][dt][r];
            }
    row_dot(P1, slot2, V(G_RZ1));
    row_dot(P2, slot2, V(G_RZ2));

    // phase 3: slot1 = Q (K stays in slot2); Q K^T, then the masked products
    stage<DK, LD>(slot1, q + tok0 * DK, (size_t)H * DK, n, tid);
    __syncthreads();
    f32x4 cQ[4];
    if constexpr (BF) cc_product_bf16(slot1, slot2, DK, cQ);
    else cc_product(slot1, slot2, DK, 1.f, cQ);
    // dGamma from A (dA o Q Khat^T) now, G_L = dL o (P Khat^T) into Cm2 for the
    // one-row shift; dA o Gamma into Cm1, dL o Gamma^- into slot0 (Vt is done)
    float* dAG = Cm1;
    float* dLG = slot0;   // C x C with row stride LDC
    float* GL = Cm2;
    f32x4 dG[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * wave + 4 * lg + r;
            const int j = 16 * jt + l16;
            const float ej = V(G_E)[j];
            const float da = j <= i ? cA[jt][r] : 0.f;
            const float dl = j < i ? cL[jt][r] : 0.f;
            dG[jt][r] = da * cQ[jt][r] * ej;
            GL[i * LDC + j] = dl * V(G_A)[i] * cK[jt][r] * ej;
            dAG[i * LDC + j] = da * Gm[i * LDC + j];
            dLG[i * LDC + j] = j < i ? dl * Gm[(i - 1) * LDC + j] : 0.f;
        }
    __syncthreads();
    // dGamma_{i,j} += G_L_{i+1,j}; the last row also gets eta_j k_j.(Vt dS'^T)_j
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * wave + 4 * lg + r;
            const int j = 16 * jt + l16;
            if (i + 1 < n) dG[jt][r] += GL[(i + 1) * LDC + j];
            if (i == n - 1 && j < n) dG[jt][r] += V(G_E)[j] * V(G_RZ1)[j];
            if (j > i || i >= n) dG[jt][r] = 0.f;
        }

    // masked products: dQ += dAG Khat;  dKhat = dAG^T Q + dLG^T P;  dP = dLG Khat
    f32x4 dKh[4][DT];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) P1[it][dt] = dKh[it][dt] = zero4();
    // k runs over the chunk rows in the k-permuted order 16 kb + 4 lg + e:
    // row reads of dAG, dLG as 16-byte vectors, column reads and the K, Q
    // rows as single values (both conflict-free with row strides 4 mod 32)
    for (int kb = 0; kb < CH / 16; ++kb) {
        float4 ag4[4], lg4[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            ag4[it] = *reinterpret_cast<const float4*>(dAG + (16 * it + l16) * LDC + 16 * kb + 4 * lg);
            lg4[it] = *reinterpret_cast<const float4*>(dLG + (16 * it + l16) * LDC + 16 * kb + 4 * lg);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int kr = 16 * kb + 4 * lg + e;
            const float ek = V(G_E)[kr];
            const float ak = V(G_A)[kr];
            float kh[DT], qv[DT], kv[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = 16 * (wave * DT + dt) + l16;
                kv[dt] = slot2[kr * LD + d];
                kh[dt] = ek * kv[dt];
                qv[dt] = slot1[kr * LD + d];
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int i = 16 * it + l16;
                const float aAG = e == 0 ? ag4[it].x : e == 1 ? ag4[it].y : e == 2 ? ag4[it].z : ag4[it].w;
                const float aLG = e == 0 ? lg4[it].x : e == 1 ? lg4[it].y : e == 2 ? lg4[it].z : lg4[it].w;
                const float aAGt = dAG[kr * LDC + i];     // dAG^T[i][k]
                const float aLGt = dLG[kr * LDC + i];     // dLG^T[i][k]
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    dQa[it][dt] = MF::mma(aAG, kh[dt], dQa[it][dt]);
                    dKh[it][dt] = MF::mma(aAGt, qv[dt], dKh[it][dt]);
                    dKh[it][dt] = MF::mma(aLGt, ak * kv[dt], dKh[it][dt]);
                    P1[it][dt] = MF::mma(aLG, kh[dt], P1[it][dt]);
                }
            }
        }
    }
    // dK += Diag(eta) dKhat + Diag(alpha) dP
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * lg + r;
                dKa[it][dt][r] += V(G_E)[i] * dKh[it][dt][r] + V(G_A)[i] * P1[it][dt][r];
            }
    // GL (Cm2) is read: reuse it for the row-dot scratch, then store dGamma there
    __syncthreads();
    row_dot(dKh, slot2, V(G_RKH));
    row_dot(P1, slot2, V(G_RP));

    // dq, dk (rows < n)
    {
        float* dqb = dq + tok0 * DK;
        float* dkb = dk + tok0 * DK;
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * it + 4 * lg + r;
                    const int d = 16 * (wave * DT + dt) + l16;
                    if (i < n) {
                        dqb[(size_t)i * H * DK + d] = dQa[it][dt][r];
                        dkb[(size_t)i * H * DK + d] = dKa[it][dt][r];
                    }
                }
    }

    // ---- coefficient gradients back to the gates ----------------------------
    float* dGm = Cm2;   // dGamma, row stride LDC
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dGm[(16 * wave + 4 * lg + r) * LDC + 16 * jt + l16] = dG[jt][r];
    // scratch, all with row stride LDC: the m table (K is done) and the
    // per-(i, j) contributions to dalpha_i, dbeta_i, dmu_i (dLG, Q and dAG
    // are done)
    float* Mt = slot2;
    float* cA_ = slot0;
    float* cS_ = slot1;
    float* cM_ = Cm1;
    __syncthreads();
    // direct terms per row
    for (int i = tid; i < CH; i += NT) {
        const float bp = i > 0 ? V(G_B)[i - 1] : 0.f;
        V(G_DAB)[i] = V(G_RX1)[i] - V(G_RY1)[i];
        V(G_DB)[i] = -V(G_RX2)[i];
        V(G_DMB)[i] = 0.f;
        // alpha: through P = Diag(alpha) K and ab1 = alpha_i b_{i-1}
        V(G_DA)[i] = V(G_RP)[i] + V(G_RY2)[i] * bp;
        // eta: through Khat and ws (wm follows with the m table)
        V(G_DE)[i] = V(G_RKH)[i] + (i < n ? Gm[(n - 1) * LDC + i] * V(G_RZ1)[i] : 0.f);
        V(G_DS)[i] = 0.f;
        V(G_DM)[i] = 0.f;
    }
    __syncthreads();
    // d(ab1)_i also reaches b_{i-1} through alpha_i; the last row's scalars
    for (int i = tid; i < n; i += NT) {
        if (i + 1 < n) V(G_DB)[i] += V(G_RY2)[i + 1] * V(G_A)[i + 1];
        if (i == n - 1) {
            V(G_DAB)[i] += scal[0];
            V(G_DB)[i] -= scal[1];
            V(G_DMB)[i] += scal[2];
        }
    }
    // m table and the column recursions (thread j < n)
    if (tid < CH) {
        const int j = tid;
        float m = 1.f;
        for (int i = 0; i < CH; ++i) {
            if (i > j) m = V(G_M)[i] * m;
            Mt[i * LDC + j] = i >= j ? m : 0.f;
            cA_[i * LDC + j] = 0.f;
            cS_[i * LDC + j] = 0.f;
            cM_[i * LDC + j] = 0.f;
        }
        if (j < n) {
            // eta_j through wm: -m_{n-1,j} k_j.(Vt dM'^T)_j
            const float dml = -V(G_E)[j] * V(G_RZ2)[j];
            float gcar = 0.f;      // dGamma_{i,j} carried down the column
            float mcar = 0.f;      // dm_{i,j} carried down the column
            for (int i = n - 1; i > j; --i) {
                const float g = dGm[i * LDC + j] + gcar;
                const float dm = (i == n - 1 ? dml : 0.f) + mcar;
                const float ai = V(G_A)[i], si = V(G_S)[i], mi = V(G_M)[i];
                const float mij = Mt[i * LDC + j];
                cA_[i * LDC + j] = g * Gm[(i - 1) * LDC + j];
                cS_[i * LDC + j] = g * mij;
                const float dmt = dm + g * si;          // total dm_{i,j}
                cM_[i * LDC + j] = dmt * Mt[(i - 1) * LDC + j];
                gcar = g * ai;
                mcar = dmt * mi;
            }
            // gamma_{j,j} = beta_j
            cS_[j * LDC + j] = dGm[j * LDC + j] + gcar;
            // the eta_j m_{n-1,j} weight: its eta part
            V(G_DE)[j] += -Mt[(n - 1) * LDC + j] * V(G_RZ2)[j];
        }
    }
    __syncthreads();
    // sum the column contributions per row, then the b, abar and mubar recursions
    for (int i = tid; i < CH; i += NT) {
        float sa = 0.f, ss = 0.f, sm = 0.f;
        for (int j = 0; j < CH; ++j) {
            sa += cA_[i * LDC + j];
            ss += cS_[i * LDC + j];
            sm += cM_[i * LDC + j];
        }
        V(G_DA)[i] += sa;
        V(G_DS)[i] += ss;
        V(G_DM)[i] += sm;
    }
    __syncthreads();
    if (wave == 0) {
        // Through b_i = alpha_i b_{i-1} + beta_i mubar_i: the total gradient of
        // b_i is db_i + alpha_{i+1} (total of b_{i+1}), a suffix recursion; then
        // abar_i = alpha_i abar_{i-1} and mubar_i = mu_i mubar_{i-1} likewise.
        // Rows >= n carry nothing (their seeds are zero and the chain is cut).
        const int i = lane;
        const bool in = i < n;
        const float anext = i + 1 < n ? V(G_A)[i + 1] : 0.f;
        const float mnext = i + 1 < n ? V(G_M)[i + 1] : 0.f;
        const float gb = suffix_affine(anext, in ? V(G_DB)[i] : 0.f, lane);
        const float bp = i > 0 ? V(G_B)[i - 1] : 0.f;
        float da = V(G_DA)[i] + gb * bp;
        const float ds = V(G_DS)[i] + gb * V(G_MB)[i];
        const float gmb0 = (in ? V(G_DMB)[i] : 0.f) + gb * V(G_S)[i];
        const float gab = suffix_affine(anext, in ? V(G_DAB)[i] : 0.f, lane);
        const float gmb = suffix_affine(mnext, in ? gmb0 : 0.f, lane);
        da += gab * (i > 0 ? V(G_AB)[i - 1] : 1.f);
        const float dm = V(G_DM)[i] + gmb * (i > 0 ? V(G_MB)[i - 1] : 1.f);
        V(G_DA)[i] = da;
        V(G_DS)[i] = ds;
        V(G_DM)[i] = dm;
    }
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
        const size_t g = tok0 + (size_t)i * H;
        dalpha[g] = V(G_DA)[i];
        deta[g] = V(G_DE)[i];
        if (dmu) dmu[g] = V(G_DM)[i];
        if (dbeta) dbeta[g] = V(G_DS)[i];
    }
}


// ---------------------------------------------------------------------------
// Per-chunk gradients for bf16 I/O: the quantities of bwd_grad_kernel (same
// formulas, same order of the coefficient recursions), laid out for eight
// wavefronts and bf16 matrix cores.
//
// Every C x DK result is computed transposed, as [d][i]: lane (l16, lg) of
// the wavefront owning d-tile dt holds d = 16 dt + 4 lg + r (r < 4) of chunk
// row i = 16 it + l16.  Then
//   * the six state products X St^T take the state rows as A operands straight
//     from registers: each wavefront loads its 16 rows of S0, M0, dS', dM'
//     once, at the start, and they also give the three inner products;
//   * the masked products take K and Q as A operands by transposing LDS
//     reads (columns of the row-major tiles), and the masked C x C matrices
//     as B operands from bf16 planes holding each value as a head and a
//     remainder (x = hi + lo to about 2^-16), formed once where the masks
//     are applied: two products per operand, fp32 sums.
// Row operands of the state products are rounded to bf16 as in
// bwd_grad_kernel (exact for dO and saved Vt); dR enters dR Vt^T as a head
// and remainder; a recomputed Vt is rounded to bf16 for its chunk products.
// C x C results: wavefront w owns row tile w % 4 and column tiles
// 2 (w / 4), 2 (w / 4) + 1.
// ---------------------------------------------------------------------------

// last-row weights of the bf16 kernel (the rows bwd_grad_kernel uses as
// scratch for them)
constexpr int G_WS = G_RED, G_WM = G_RED + 1;

// x rounded to bf16 (nearest even), two per 32-bit word
__device__ __forceinline__ unsigned bwd_pack_bf16(float a, float b)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_bit_cast(unsigned, bf16x2{static_cast<__bf16>(a), static_cast<__bf16>(b)});
}
// Column of the masked-operand planes holding chunk row k: inside each 32
// columns, the k order of a 16x16x32 step whose lane group g takes rows
// 32 p + 4 g .. + 3 and 32 p + 16 + 4 g .. + 3, so that they are 8 adjacent
// columns.
__device__ __forceinline__ int kperm(int k)
{
    return (k & ~31) | ((k & 12) << 1) | ((k & 16) >> 2) | (k & 3);
}

// a if c else b, on values (a conditional between two named vectors would
// select between their addresses and put both in memory)
__device__ __forceinline__ uint4 sel4(bool c, uint4 a, uint4 b)
{
    return uint4{c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w};
}

// value of x in lane l (l uniform)
__device__ __forceinline__ float readlane_f(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ bf16x8 bwd_cat8(const bf16x4& a, const bf16x4& b)
{
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Sum over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48), in every
// lane, without a trip through LDS: permlane16_swap of a value with itself
// exchanges groups 1 and 0 and groups 3 and 2 between its two results, so
// their sum holds p0 + p1 in groups 0, 1 and p2 + p3 in groups 2, 3;
// permlane32_swap does the same with the halves.
__device__ __forceinline__ float bwd_sum_groups(float p)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p), false,
                                                    false);
    const float q = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(q), __float_as_uint(q), false,
                                                    false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
// x of the lane d places further round its row of 16 (DPP row_ror:d)
__device__ __forceinline__ float bwd_row_ror(float x, int d)
{
    int r = __float_as_int(x);
    switch (d) {
    case 1: r = __builtin_amdgcn_mov_dpp(r, 0x121, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_mov_dpp(r, 0x122, 0xf, 0xf, false); break;
    case 4: r = __builtin_amdgcn_mov_dpp(r, 0x124, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_mov_dpp(r, 0x128, 0xf, 0xf, false); break;
    }
    return __int_as_float(r);
}
// Sum over the 64 lanes, in every lane.
__device__ __forceinline__ float bwd_sum_wave(float p)
{
    p += bwd_row_ror(p, 8);
    p += bwd_row_ror(p, 4);
    p += bwd_row_ror(p, 2);
    p += bwd_row_ror(p, 1);
    return bwd_sum_groups(p);
}

// x of lane i - d (row_shr) or i + d (row_shl) of the lane's row of 16; lanes
// whose source lies outside the row take `fill` (DPP)
__device__ __forceinline__ float bwd_row_shr(float x, int d, float fill)
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
__device__ __forceinline__ float bwd_row_shl(float x, int d, float fill)
{
    int r = __float_as_int(fill);
    switch (d) {
    case 1: r = __builtin_amdgcn_update_dpp(r, __float_as_int(x), 0x101, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(r, __float_as_int(x), 0x102, 0xf, 0xf, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(r, __float_as_int(x), 0x104, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_update_dpp(r, __float_as_int(x), 0x108, 0xf, 0xf, false); break;
    }
    return __int_as_float(r);
}
// The scans of prefix_affine and suffix_affine (lane i holding row i) with
// the shuffles replaced: four DPP steps inside each row of 16 lanes, then the
// rows composed from the values at their ends (read as uniform values) --
// prefix: x_i = m_i x_{i-1} + c_i from x_{-1} = 0; suffix: y_i = c_i + m_i y_{i+1}
// from y_64 = 0.  Each within-row step composes the lane's map with the one
// of the d rows before (after) it, as the shuffle scans do.
__device__ __forceinline__ float bwd_prefix_affine(float m, float c, int lane)
{
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
        const float mp = bwd_row_shr(m, d, 1.f), cp = bwd_row_shr(c, d, 0.f);
        c = m * cp + c;
        m = m * mp;
    }
    // x entering rows 1, 2, 3 (the map of row r at its last lane 16 r + 15)
    const float x1 = readlane_f(c, 15);
    const float x2 = readlane_f(m, 31) * x1 + readlane_f(c, 31);
    const float x3 = readlane_f(m, 47) * x2 + readlane_f(c, 47);
    const int r = lane >> 4;
    const float xin = r == 0 ? 0.f : r == 1 ? x1 : r == 2 ? x2 : x3;
    return m * xin + c;
}
__device__ __forceinline__ float bwd_suffix_affine(float m, float c, int lane)
{
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
        const float mn = bwd_row_shl(m, d, 1.f), cn = bwd_row_shl(c, d, 0.f);
        c = c + m * cn;
        m = m * mn;
    }
    // y at the first lanes of rows 3, 2, 1 (the map of row r at lane 16 r)
    const float y3 = readlane_f(c, 48);
    const float y2 = readlane_f(m, 32) * y3 + readlane_f(c, 32);
    const float y1 = readlane_f(m, 16) * y2 + readlane_f(c, 16);
    const int r = lane >> 4;
    const float yout = r == 3 ? 0.f : r == 2 ? y3 : r == 1 ? y2 : y1;
    return m * yout + c;
}
// inclusive prefix products of a and b over the 64 lanes
__device__ __forceinline__ void bwd_prefix_prod2(float& a, float& b, int lane)
{
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
        a *= bwd_row_shr(a, d, 1.f);
        b *= bwd_row_shr(b, d, 1.f);
    }
    const float a0 = readlane_f(a, 15), a1 = a0 * readlane_f(a, 31), a2 = a1 * readlane_f(a, 47);
    const float b0 = readlane_f(b, 15), b1 = b0 * readlane_f(b, 31), b2 = b1 * readlane_f(b, 47);
    const int r = lane >> 4;
    a *= r == 0 ? 1.f : r == 1 ? a0 : r == 2 ? a1 : a2;
    b *= r == 0 ? 1.f : r == 1 ? b0 : r == 2 ? b1 : b2;
}

constexpr int NT8 = 512;

template <int DK, int DV>
struct GradBfSmem {
    static constexpr int LQ = DK + 8;   // bf16 row stride of Q, K (16-byte pad)
    static constexpr int LV = DV + 8;   // bf16 row stride of dO, Vt
    static constexpr int LR = DV + 4;   // fp32 row stride of dR
    static constexpr int LDC = CH + 4;  // fp32 row stride of C x C matrices
    static constexpr int LP = CH + 8;   // bf16 row stride of a C x C plane
    static constexpr int CM = CH * LDC * 4;       // bytes of one fp32 C x C matrix
    static constexpr int PLANE = CH * LP * 2;     // bytes of one bf16 C x C plane
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = OFF_Q + CH * LQ * 2;
    static constexpr int OFF_DO = OFF_K + CH * LQ * 2;
    static constexpr int OFF_VT = OFF_DO + CH * LV * 2;
    static constexpr int OFF_DR = OFF_VT + CH * LV * 2;
    static constexpr int END_TILES = OFF_DR + CH * LR * 4;
    // the tiles' area also holds seven of the eight bf16 planes of the masked
    // operands (from the dO tile on) once the chunk products are done
    static constexpr int END_A = END_TILES > OFF_DO + 7 * PLANE ? END_TILES : OFF_DO + 7 * PLANE;
    static constexpr int OFF_GM = END_A;          // Gamma
    static constexpr int OFF_C1 = OFF_GM + CM;    // m, then planes
    static constexpr int OFF_C2 = OFF_C1 + CM;    // row-dot partials, G_L, dGamma
    static constexpr int OFF_VEC = OFF_C2 + CM;
    static constexpr int NV = 24;
    static constexpr int BYTES = OFF_VEC + (NV * CH + 32) * 4;
    static constexpr int OFF_PL = OFF_DO;
    static_assert(PLANE <= CM, "the eighth plane goes to C1");
};

// plane p of the masked operands: 0/1 dAG o eta (hi, lo), 2/3 dAG^T,
// 4/5 (alpha dLG)^T, 6/7 dLG o eta
template <int DK, int DV>
__device__ __forceinline__ int plane_off(int p)
{
    using SM = GradBfSmem<DK, DV>;
    // seven in the tiles' area after Q and K, the last in C1 (free once the
    // m table has given the last-row weights)
    return p < 7 ? SM::OFF_PL + p * SM::PLANE : SM::OFF_C1;
}

// SAVED: the forward saved the residuals (Vsaved, bf16 tokens); otherwise
// the re-scan wrote them in fp32 to Vts.
template <int DK, int DV, bool SAVED>
__global__ __launch_bounds__(NT8) void bwd_grad_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ dO,
    const float* __restrict__ dv, const float* __restrict__ Vts, const __bf16* __restrict__ Vsaved,
    const __bf16* __restrict__ Hs, const __bf16* __restrict__ Hd, const float* __restrict__ alpha,
    const float* __restrict__ mu, const float* __restrict__ eta, const float* __restrict__ beta,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dalpha,
    float* __restrict__ dmu, float* __restrict__ deta, float* __restrict__ dbeta,
    const float* S0x, const float* M0x, const float* dSTx, const float* dMTx, int T, int H,
    int NC)
{
    using SM = GradBfSmem<DK, DV>;
    using BM = Mma<__bf16>;
    constexpr int LQ = SM::LQ, LV = SM::LV, LR = SM::LR, LDC = SM::LDC, LP = SM::LP;
    constexpr int NDT = DK / 16;             // d-tiles: 8 or 4
    constexpr int NIT = 4 * NDT / 8;         // row tiles per wavefront: 4 or 2
    constexpr int KSV = DV / 32;             // 32-column k-steps over DV
    constexpr int KSK = DK / 32;             // ... over DK
    static_assert(NDT == 8 || NDT == 4, "head size");
    __shared__ __align__(16) char smem[SM::BYTES];
    __bf16* Qs = reinterpret_cast<__bf16*>(smem + SM::OFF_Q);
    __bf16* Ks = reinterpret_cast<__bf16*>(smem + SM::OFF_K);
    __bf16* dOs = reinterpret_cast<__bf16*>(smem + SM::OFF_DO);
    __bf16* Vs = reinterpret_cast<__bf16*>(smem + SM::OFF_VT);
    float* dRs = reinterpret_cast<float*>(smem + SM::OFF_DR);
    float* Gm = reinterpret_cast<float*>(smem + SM::OFF_GM);
    float* Cm1 = reinterpret_cast<float*>(smem + SM::OFF_C1);
    float* Cm2 = reinterpret_cast<float*>(smem + SM::OFF_C2);
    float* vec = reinterpret_cast<float*>(smem + SM::OFF_VEC);
    float* scal = vec + SM::NV * CH;     // 3 inner products, then 3 x 8 partials
    auto V = [&](int row) { return vec + row * CH; };
    auto plane = [&](int p) { return reinterpret_cast<__bf16*>(smem + plane_off<DK, DV>(p)); };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int c = (int)(blockIdx.x % NC);
    const int bh = (int)(blockIdx.x / NC);
    const int h = bh % H;
    const int b = bh / H;
    const int t0 = c * CH;
    const int n = min(CH, T - t0);
    const size_t tok0 = ((size_t)b * T + t0) * H + h;
    const size_t chn = (size_t)bh * NC + c;
    const int dt = wave % NDT;               // this wavefront's d-tile
    const int it0 = (wave / NDT) * NIT;      // ... and first row tile
    const bool owner = wave < NDT;           // counts the inner products once

    // ---- loads: the chunk's tiles, then this wavefront's state rows --------
    // (issued last, so that the tiles' waits leave them in flight: they are
    // first used by the state products)
    // state row d = 16 dt + l16, columns 32 s + 8 lg .. + 7: an A fragment
    uint4 st[4][KSV];
    // the chunk's rows into LDS: bf16 tiles as bf16 (a recomputed fp32 Vt is
    // rounded), dR as fp32; rows >= n are zero
    {
        constexpr int PQ = CH * DK / 8 / NT8;    // 16-byte pieces per thread
        constexpr int PV = CH * DV / 8 / NT8;
        constexpr int PR = CH * DV / 4 / NT8;
        static_assert(PQ >= 1 && PV >= 1 && PR >= 1, "tiles split over the workgroup");
        uint4 bq[PQ], bk[PQ], bo[PV], bvt[SAVED ? PV : 1], bvf[SAVED ? 1 : 2 * PV];
        float4 br[PR];
        // every load is unconditional (rows >= n read row n - 1 and are zeroed
        // when stored): a load under a branch makes the compiler wait for all
        // outstanding loads where the branches join
        const int nl = n - 1;
#pragma unroll
        for (int u = 0; u < PQ; ++u) {
            const int idx = tid + u * NT8, row = min(idx / (DK / 8), nl), c8 = idx % (DK / 8);
            const size_t g = (tok0 + (size_t)row * H) * DK + 8 * c8;
            bq[u] = *reinterpret_cast<const uint4*>(q + g);
            bk[u] = *reinterpret_cast<const uint4*>(k + g);
        }
#pragma unroll
        for (int u = 0; u < PV; ++u) {
            const int idx = tid + u * NT8, row = min(idx / (DV / 8), nl), c8 = idx % (DV / 8);
            const size_t g = (tok0 + (size_t)row * H) * DV + 8 * c8;
            bo[u] = *reinterpret_cast<const uint4*>(dO + g);
            if constexpr (SAVED) {
                bvt[u] = *reinterpret_cast<const uint4*>(Vsaved + g);
            } else {
                const float* src = Vts + (chn * CH + row) * DV + 8 * c8;
                bvf[2 * u] = *reinterpret_cast<const uint4*>(src);
                bvf[2 * u + 1] = *reinterpret_cast<const uint4*>(src + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < PR; ++u) {
            const int idx = tid + u * NT8, row = min(idx / (DV / 4), nl), c4 = idx % (DV / 4);
            br[u] = *reinterpret_cast<const float4*>(dv + (tok0 + (size_t)row * H) * DV + 4 * c4);
        }
        // gates of row lane (rows >= n: alpha 1, mu, eta, beta 0)
        float ga_, gm_ = 0.f, ge_, gs_ = 1.f;
        {
            const size_t g = tok0 + (size_t)min(lane, nl) * H;
            ga_ = alpha[g];
            ge_ = eta[g];
            if (mu) gm_ = mu[g];
            if (beta) gs_ = beta[g];
        }
        {
            const __bf16* S0 = Hs + chn * 2 * DK * DV;
            const __bf16* Sd = Hd + chn * 2 * DK * DV;
            const __bf16* base[4] = {S0, S0 + DK * DV, Sd, Sd + DK * DV};   // S0, M0, dS', dM'
            const int d = 16 * dt + l16;
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int s = 0; s < KSV; ++s)
                    st[x][s] = *reinterpret_cast<const uint4*>(base[x] + (size_t)d * DV + 32 * s + 8 * lg);
        }
        if (tid < CH) {
            const bool in = lane < n;
            V(G_A)[lane] = in ? ga_ : 1.f;
            V(G_M)[lane] = in ? gm_ : 0.f;
            V(G_E)[lane] = in ? ge_ : 0.f;
            V(G_S)[lane] = in ? gs_ : 0.f;
        }
        const uint4 z4 = uint4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < PQ; ++u) {
            const int idx = tid + u * NT8, row = idx / (DK / 8), c8 = idx % (DK / 8);
            const bool in = row < n;
            *reinterpret_cast<uint4*>(Qs + row * LQ + 8 * c8) = sel4(in, bq[u], z4);
            *reinterpret_cast<uint4*>(Ks + row * LQ + 8 * c8) = sel4(in, bk[u], z4);
        }
#pragma unroll
        for (int u = 0; u < PV; ++u) {
            const int idx = tid + u * NT8, row = idx / (DV / 8), c8 = idx % (DV / 8);
            const bool in = row < n;
            *reinterpret_cast<uint4*>(dOs + row * LV + 8 * c8) = sel4(in, bo[u], z4);
            if constexpr (SAVED) {
                *reinterpret_cast<uint4*>(Vs + row * LV + 8 * c8) = sel4(in, bvt[u], z4);
            } else {
                const uint4 a = bvf[2 * u], e = bvf[2 * u + 1];
                const uint4 w = uint4{bwd_pack_bf16(__uint_as_float(a.x), __uint_as_float(a.y)),
                                      bwd_pack_bf16(__uint_as_float(a.z), __uint_as_float(a.w)),
                                      bwd_pack_bf16(__uint_as_float(e.x), __uint_as_float(e.y)),
                                      bwd_pack_bf16(__uint_as_float(e.z), __uint_as_float(e.w))};
                *reinterpret_cast<uint4*>(Vs + row * LV + 8 * c8) = sel4(in, w, z4);
            }
        }
#pragma unroll
        for (int u = 0; u < PR; ++u) {
            const int idx = tid + u * NT8, row = idx / (DV / 4), c4 = idx % (DV / 4);
            *reinterpret_cast<float4*>(dRs + row * LR + 4 * c4) =
                row < n ? br[u] : float4{0.f, 0.f, 0.f, 0.f};
        }
    }
    for (int i = tid; i < (SM::NV - G_RX1) * CH; i += NT8) vec[G_RX1 * CH + i] = 0.f;
    lds_barrier();

    // ---- coefficients: abar, mubar, b; Gamma and m by columns ---------------
    if (wave == 0) {
        const float a = V(G_A)[lane], m = V(G_M)[lane];
        float pa = a, pm = m;
        bwd_prefix_prod2(pa, pm, lane);
        V(G_AB)[lane] = pa;
        V(G_MB)[lane] = pm;
        V(G_B)[lane] = bwd_prefix_affine(a, V(G_S)[lane] * pm, lane);
    }
    {
        // Gamma and m by 8-row blocks: wavefront I runs rows 8 I ..
        // 8 I + 7 of every column j = lane from zero at the block's start
        // (m gets 1 added on the diagonal row, which starts column j there
        // and leaves the rows above it zero), with the gates of row i from
        // lane i's registers, and stores these block-local values; the
        // response of row i to the values (m0, g0) entering its block,
        // m0 rp and g0 ra + m0 rg, is the same for every column and goes to
        // a row table, the block's exits to the exchange (both in C2).
        const int I = wave, j = lane;
        const float ga = V(G_A)[lane], gm = V(G_M)[lane], gs = V(G_S)[lane];
        float* xch = Cm2;   // 0: m exits, 512: Gamma exits, 1024 + 4 i: row responses
        float m = 0.f, g = 0.f, rp = 1.f, ra = 1.f, rg = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int i = 8 * I + t;
            const float ai = readlane_f(ga, i), mi = readlane_f(gm, i), si = readlane_f(gs, i);
            m = mi * m + (i == j ? 1.f : 0.f);
            g = ai * g + si * m;
            Gm[i * LDC + j] = g;
            Cm1[i * LDC + j] = m;
            rp = mi * rp;
            rg = ai * rg + si * rp;
            ra = ai * ra;
            if (lane == 0) {
                xch[1024 + 4 * i] = rp;
                xch[1025 + 4 * i] = ra;
                xch[1026 + 4 * i] = rg;
            }
        }
        xch[64 * I + j] = m;
        xch[512 + 64 * I + j] = g;
    }
    lds_barrier();
    {
        // the values entering block I, composed from the exits of the blocks
        // above it; then their response on every row of the block
        const int I = wave, j = lane;
        const float* xch = Cm2;
        float m0 = 0.f, g0 = 0.f;
        for (int K = 0; K < I; ++K) {
            const int e = 1024 + 4 * (8 * K + 7);
            const float mn = xch[64 * K + j] + m0 * xch[e];
            g0 = xch[512 + 64 * K + j] + g0 * xch[e + 1] + m0 * xch[e + 2];
            m0 = mn;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int i = 8 * I + t;
            const float4 r = *reinterpret_cast<const float4*>(xch + 1024 + 4 * i);
            Gm[i * LDC + j] += g0 * r.y + m0 * r.z;
            Cm1[i * LDC + j] += m0 * r.x;
        }
    }
    lds_barrier();
    // last-row weights ws_j = eta_j gamma_{n-1,j}, wm_j = eta_j m_{n-1,j}
    if (tid < CH) {
        const int j = tid;
        V(G_WS)[j] = V(G_E)[j] * Gm[(n - 1) * LDC + j];
        V(G_WM)[j] = V(G_E)[j] * Cm1[(n - 1) * LDC + j];
    }
    lds_barrier();

    // the three inner products <dS', S0>, <dS', M0>, <dM', M0> from the
    // registers (each state element counted by one wavefront); summed with
    // the row dots.  The first chunk's entry state and the last chunk's
    // exit-state gradients are the call's own fp32 inputs (S0, M0, dS_T,
    // dM_T; the stored copies are rounded to bf16): there the sums take them
    // as they are.  A sum over d_k d_v products of two rounded states carries
    // a rounding error of about 2^-9 sqrt(d_k d_v) rms(dS') rms(S0), which
    // for a short sequence is a large part of the gate gradients themselves.
    {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f;
        const float* xS = c == 0 ? S0x : nullptr;
        const float* xM = c == 0 ? M0x : nullptr;
        const float* xdS = c == NC - 1 ? dSTx : nullptr;
        const float* xdM = c == NC - 1 ? dMTx : nullptr;
        if (owner && (xS || xM || xdS || xdM)) {
            // row 16 dt + l16 of the state, columns 32 s + 8 lg .. + 7
            const size_t so = (size_t)bh * DK * DV + (size_t)(16 * dt + l16) * DV + 8 * lg;
#pragma unroll
            for (int s = 0; s < KSV; ++s) {
                float v[4][8];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const unsigned w[4] = {st[x][s].x, st[x][s].y, st[x][s].z, st[x][s].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[x][2 * e] = __uint_as_float(w[e] << 16);
                        v[x][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
                    }
                }
                const float* xp[4] = {xS, xM, xdS, xdM};
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    if (xp[x]) {
                        const float4 lo = *reinterpret_cast<const float4*>(xp[x] + so + 32 * s);
                        const float4 hi = *reinterpret_cast<const float4*>(xp[x] + so + 32 * s + 4);
                        v[x][0] = lo.x, v[x][1] = lo.y, v[x][2] = lo.z, v[x][3] = lo.w;
                        v[x][4] = hi.x, v[x][5] = hi.y, v[x][6] = hi.z, v[x][7] = hi.w;
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    a0 += v[2][j] * v[0][j];
                    a1 += v[2][j] * v[1][j];
                    a2 += v[3][j] * v[1][j];
                }
            }
        } else if (owner) {
#pragma unroll
            for (int s = 0; s < KSV; ++s) {
                const unsigned w0[4] = {st[0][s].x, st[0][s].y, st[0][s].z, st[0][s].w};
                const unsigned w1[4] = {st[1][s].x, st[1][s].y, st[1][s].z, st[1][s].w};
                const unsigned w2[4] = {st[2][s].x, st[2][s].y, st[2][s].z, st[2][s].w};
                const unsigned w3[4] = {st[3][s].x, st[3][s].y, st[3][s].z, st[3][s].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float s0a = __uint_as_float(w0[e] << 16), s0b = __uint_as_float(w0[e] & 0xffff0000u);
                    const float m0a = __uint_as_float(w1[e] << 16), m0b = __uint_as_float(w1[e] & 0xffff0000u);
                    const float dsa = __uint_as_float(w2[e] << 16), dsb = __uint_as_float(w2[e] & 0xffff0000u);
                    const float dma = __uint_as_float(w3[e] << 16), dmb = __uint_as_float(w3[e] & 0xffff0000u);
                    a0 += dsa * s0a + dsb * s0b;
                    a1 += dsa * m0a + dsb * m0b;
                    a2 += dma * m0a + dmb * m0b;
                }
            }
        }
        a0 = bwd_sum_wave(a0);
        a1 = bwd_sum_wave(a1);
        a2 = bwd_sum_wave(a2);
        if (lane == 0) {
            scal[8 + wave] = a0;
            scal[16 + wave] = a1;
            scal[24 + wave] = a2;
        }
    }
    // ---- state products, transposed: P[x]^T = St X^T ----------------------
    // (P1 dO S0^T, P2 dO M0^T, P3 dR S0^T, P4 dR M0^T, P5 Vt dS'^T, P6 Vt dM'^T)
    f32x4 P[6][NIT];
#pragma unroll
    for (int x = 0; x < 6; ++x)
#pragma unroll
        for (int u = 0; u < NIT; ++u) P[x][u] = zero4();
#pragma unroll
    for (int s = 0; s < KSV; ++s) {
        const bf16x8 aS0 = __builtin_bit_cast(bf16x8, st[0][s]);
        const bf16x8 aM0 = __builtin_bit_cast(bf16x8, st[1][s]);
        const bf16x8 adS = __builtin_bit_cast(bf16x8, st[2][s]);
        const bf16x8 adM = __builtin_bit_cast(bf16x8, st[3][s]);
#pragma unroll
        for (int u = 0; u < NIT; ++u) {
            const int i = 16 * (it0 + u) + l16;
            const bf16x8 bO = *reinterpret_cast<const bf16x8*>(dOs + i * LV + 32 * s + 8 * lg);
            const bf16x8 bV = *reinterpret_cast<const bf16x8*>(Vs + i * LV + 32 * s + 8 * lg);
            const float4 r0 = *reinterpret_cast<const float4*>(dRs + i * LR + 32 * s + 8 * lg);
            const float4 r1 = *reinterpret_cast<const float4*>(dRs + i * LR + 32 * s + 8 * lg + 4);
            const bf16x8 bR = __builtin_bit_cast(
                bf16x8, uint4{bwd_pack_bf16(r0.x, r0.y), bwd_pack_bf16(r0.z, r0.w), bwd_pack_bf16(r1.x, r1.y),
                              bwd_pack_bf16(r1.z, r1.w)});
            P[0][u] = BM::mma(aS0, bO, P[0][u]);
            P[1][u] = BM::mma(aM0, bO, P[1][u]);
            P[2][u] = BM::mma(aS0, bR, P[2][u]);
            P[3][u] = BM::mma(aM0, bR, P[3][u]);
            P[4][u] = BM::mma(adS, bV, P[4][u]);
            P[5][u] = BM::mma(adM, bV, P[5][u]);
        }
    }
    // dQ, dK state parts and the six row dots (q with P1, P2; k with P3..P6),
    // partial over this d-tile: red[x][dt][i] in C2
    float* red = Cm2;
    f32x4 dQa[NIT], dKa[NIT];
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
        const int i = 16 * (it0 + u) + l16;
        const float ab = V(G_AB)[i], bb = V(G_B)[i];
        const float ab1 = i > 0 ? V(G_A)[i] * V(G_B)[i - 1] : 0.f;
        const float wsv = V(G_WS)[i], wmv = V(G_WM)[i];
        dQa[u] = ab * P[0][u] - bb * P[1][u];
        dKa[u] = -ab * P[2][u] + ab1 * P[3][u] + wsv * P[4][u] - wmv * P[5][u];
        const bf16x4 qd = *reinterpret_cast<const bf16x4*>(Qs + i * LQ + 16 * dt + 4 * lg);
        const bf16x4 kd = *reinterpret_cast<const bf16x4*>(Ks + i * LQ + 16 * dt + 4 * lg);
#pragma unroll
        for (int x = 0; x < 6; ++x) {
            const bf16x4 y = x < 2 ? qd : kd;
            float p = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) p += P[x][u][r] * static_cast<float>(y[r]);
            p = bwd_sum_groups(p);
            if (lg == 0) red[(x * NDT + dt) * CH + i] = p;
        }
    }

    // ---- chunk products (row tile rw, column tiles cw, cw + 1) -------------
    const int rw = wave & 3, cw = 2 * (wave >> 2);
    f32x4 cA[2], cL[2], cK[2], cQ[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) cA[e] = cL[e] = cK[e] = cQ[e] = zero4();
    {
        const int ia = 16 * rw + l16;
#pragma unroll
        for (int s = 0; s < KSV; ++s) {
            const bf16x8 aO = *reinterpret_cast<const bf16x8*>(dOs + ia * LV + 32 * s + 8 * lg);
            const float4 r0 = *reinterpret_cast<const float4*>(dRs + ia * LR + 32 * s + 8 * lg);
            const float4 r1 = *reinterpret_cast<const float4*>(dRs + ia * LR + 32 * s + 8 * lg + 4);
            // -dR as a bf16 head and remainder
            const float rr[8] = {-r0.x, -r0.y, -r0.z, -r0.w, -r1.x, -r1.y, -r1.z, -r1.w};
            bf16x8 rh, rl;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                rh[j] = static_cast<__bf16>(rr[j]);
                rl[j] = static_cast<__bf16>(rr[j] - static_cast<float>(rh[j]));
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int jb = 16 * (cw + e) + l16;
                const bf16x8 bV = *reinterpret_cast<const bf16x8*>(Vs + jb * LV + 32 * s + 8 * lg);
                cA[e] = BM::mma(aO, bV, cA[e]);
                cL[e] = BM::mma(rh, bV, cL[e]);
                cL[e] = BM::mma(rl, bV, cL[e]);
            }
        }
#pragma unroll
        for (int s = 0; s < KSK; ++s) {
            const bf16x8 aK = *reinterpret_cast<const bf16x8*>(Ks + ia * LQ + 32 * s + 8 * lg);
            const bf16x8 aQ = *reinterpret_cast<const bf16x8*>(Qs + ia * LQ + 32 * s + 8 * lg);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int jb = 16 * (cw + e) + l16;
                const bf16x8 bK = *reinterpret_cast<const bf16x8*>(Ks + jb * LQ + 32 * s + 8 * lg);
                cK[e] = BM::mma(aK, bK, cK[e]);
                cQ[e] = BM::mma(aQ, bK, cQ[e]);
            }
        }
    }
    lds_barrier();   // red complete; dO, Vt, dR read for the last time
    for (int i = tid; i < 6 * CH; i += NT8) {
        const int x = i / CH, r = i % CH;
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < NDT; ++u) sum += red[(x * NDT + u) * CH + r];
        V(G_RX1 + x)[r] = sum;   // RX1, RX2, RY1, RY2, RZ1, RZ2 are consecutive rows
    }
    if (tid < 3) {
        const float* p = scal + 8 * (tid + 1);
        scal[tid] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }
    lds_barrier();   // red consumed: C2 free for G_L

    // ---- masks: dGamma, G_L, and the masked operands as bf16 planes --------
    float* GL = Cm2;
    f32x4 dG[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * rw + 4 * lg + r;
            const int j = 16 * (cw + e) + l16;
            const float ej = V(G_E)[j], ai = V(G_A)[i];
            const float da = j <= i ? cA[e][r] : 0.f;
            const float dl = j < i ? cL[e][r] : 0.f;
            dG[e][r] = da * cQ[e][r] * ej;
            GL[i * LDC + j] = dl * ai * cK[e][r] * ej;
            const float dag = da * Gm[i * LDC + j];
            const float dlg = j < i ? dl * Gm[(i - 1) * LDC + j] : 0.f;
            // x = hi + lo for each of the four operands
            const float xs[4] = {dag * ej, dag, ai * dlg, dlg * ej};
            const int rowp[4] = {i, j, j, i};
            const int colp[4] = {j, i, i, j};
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                const __bf16 hi = static_cast<__bf16>(xs[o]);
                const __bf16 lo = static_cast<__bf16>(xs[o] - static_cast<float>(hi));
                const int cp = kperm(colp[o]);
                plane(2 * o)[rowp[o] * LP + cp] = hi;
                plane(2 * o + 1)[rowp[o] * LP + cp] = lo;
            }
        }
    lds_barrier();
    // dGamma_{i,j} += G_L_{i+1,j}; the last row also gets eta_j k_j.(Vt dS'^T)_j
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * rw + 4 * lg + r;
            const int j = 16 * (cw + e) + l16;
            if (i + 1 < n) dG[e][r] += GL[(i + 1) * LDC + j];
            if (i == n - 1 && j < n) dG[e][r] += V(G_E)[j] * V(G_RZ1)[j];
            if (j > i || i >= n) dG[e][r] = 0.f;
        }

    // ---- masked products, transposed, k over the chunk rows ---------------
    //   dQ^T   += K^T (dAG o eta)^T          dKh^T = Q^T dAG + K^T (alpha dLG)
    //   dP^T    = K^T (dLG o eta)^T
    // A: columns d of K, Q by transposing reads (k order 32 p + 4 lg + j and
    // 32 p + 16 + 4 lg + j); B: row i of the planes in the same k order.
    f32x4 dKh[NIT], dPa[NIT];
#pragma unroll
    for (int u = 0; u < NIT; ++u) dKh[u] = dPa[u] = zero4();
    {
        const int trow = 4 * lg + (l16 >> 2), tcol = 16 * dt + 4 * (l16 & 3);
        const char* kt = reinterpret_cast<const char*>(Ks + trow * LQ + tcol);
        const char* qt = reinterpret_cast<const char*>(Qs + trow * LQ + tcol);
        constexpr int R16 = 16 * LQ * 2;   // 16 rows further, bytes
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const bf16x8 aK = bwd_cat8(lds_read_tr4(kt + 2 * p * R16), lds_read_tr4(kt + (2 * p + 1) * R16));
            const bf16x8 aQ = bwd_cat8(lds_read_tr4(qt + 2 * p * R16), lds_read_tr4(qt + (2 * p + 1) * R16));
#pragma unroll
            for (int u = 0; u < NIT; ++u) {
                const int i = 16 * (it0 + u) + l16;
                // columns stored in k order: one 16-byte read per fragment
                auto bfr = [&](int pl) {
                    return *reinterpret_cast<const bf16x8*>(plane(pl) + i * LP + 32 * p + 8 * lg);
                };
                dQa[u] = BM::mma(aK, bfr(0), dQa[u]);
                dQa[u] = BM::mma(aK, bfr(1), dQa[u]);
                dKh[u] = BM::mma(aQ, bfr(2), dKh[u]);
                dKh[u] = BM::mma(aQ, bfr(3), dKh[u]);
                dKh[u] = BM::mma(aK, bfr(4), dKh[u]);
                dKh[u] = BM::mma(aK, bfr(5), dKh[u]);
                dPa[u] = BM::mma(aK, bfr(6), dPa[u]);
                dPa[u] = BM::mma(aK, bfr(7), dPa[u]);
            }
        }
    }
    lds_barrier();   // G_L read: C2 takes the last row-dot partials
    // dK += Diag(eta) dKhat + Diag(alpha) dP; row dots k.dKhat, k.dP
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
        const int i = 16 * (it0 + u) + l16;
        dKa[u] += V(G_E)[i] * dKh[u] + V(G_A)[i] * dPa[u];
        const bf16x4 kd = *reinterpret_cast<const bf16x4*>(Ks + i * LQ + 16 * dt + 4 * lg);
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p0 += dKh[u][r] * static_cast<float>(kd[r]);
            p1 += dPa[u][r] * static_cast<float>(kd[r]);
        }
        p0 = bwd_sum_groups(p0);
        p1 = bwd_sum_groups(p1);
        if (lg == 0) {
            red[(0 * NDT + dt) * CH + i] = p0;
            red[(1 * NDT + dt) * CH + i] = p1;
        }
        // dq, dk rows < n: 4 consecutive d per lane
        if (i < n) {
            const size_t g = (tok0 + (size_t)i * H) * DK + 16 * dt + 4 * lg;
            *reinterpret_cast<f32x4*>(dq + g) = dQa[u];
            *reinterpret_cast<f32x4*>(dk + g) = dKa[u];
        }
    }
    lds_barrier();
    for (int i = tid; i < 2 * CH; i += NT8) {
        const int x = i / CH, r = i % CH;
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < NDT; ++u) sum += red[(x * NDT + u) * CH + r];
        V(x == 0 ? G_RKH : G_RP)[r] = sum;
    }
    lds_barrier();

    // ---- coefficient gradients back to the gates (as in bwd_grad_kernel) ---
    float* dGm = Cm2;   // dGamma, row stride LDC
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dGm[(16 * rw + 4 * lg + r) * LDC + 16 * (cw + e) + l16] = dG[e][r];
    // scratch with row stride LDC in the tiles' area (all read by now)
    float* cA_ = reinterpret_cast<float*>(smem);
    float* cS_ = cA_ + CH * LDC;
    float* cM_ = cS_ + CH * LDC;
    static_assert(4 * SM::CM <= SM::END_A, "tail scratch");
    for (int i = tid; i < CH; i += NT8) {
        const float bp = i > 0 ? V(G_B)[i - 1] : 0.f;
        V(G_DAB)[i] = V(G_RX1)[i] - V(G_RY1)[i];
        V(G_DB)[i] = -V(G_RX2)[i];
        V(G_DMB)[i] = 0.f;
        V(G_DA)[i] = V(G_RP)[i] + V(G_RY2)[i] * bp;
        V(G_DE)[i] = V(G_RKH)[i] + (i < n ? Gm[(n - 1) * LDC + i] * V(G_RZ1)[i] : 0.f);
        V(G_DS)[i] = 0.f;
        V(G_DM)[i] = 0.f;
    }
    lds_barrier();
    for (int i = tid; i < n; i += NT8) {
        if (i + 1 < n) V(G_DB)[i] += V(G_RY2)[i + 1] * V(G_A)[i + 1];
        if (i == n - 1) {
            V(G_DAB)[i] += scal[0];
            V(G_DB)[i] -= scal[1];
            V(G_DMB)[i] += scal[2];
        }
    }
    // Column j of the recursions back through Gamma and m, by 8-row blocks
    // as the forward ones: wavefront I takes rows 8 I .. 8 I + 7 of every
    // column.  Going up the rows, with the carries (gcar, mcar) coming
    // from row i + 1:
    //   g = dGamma_{i,j} + gcar,  dmt = [i = n - 1] dml + mcar + beta_i g,
    //   gcar <- alpha_i g,  mcar <- mu_i dmt
    // on the rows j < i < n, and the contributions g Gamma_{i-1,j} (to
    // dalpha_i), g m_{i,j} (to dbeta_i), dmt m_{i-1,j} (to dmu_i).  Each
    // block runs from zero carries; the carries entering it are composed
    // from the exits of the blocks below it in row order (above it in the
    // recursion), and their response on the block's rows is the same for
    // every column.  m is rebuilt the same way, going down.
    // Pass 1 keeps the block-local values of m, g and dmt in the scratch
    // (cS_, cA_, cM_ at their own (i, j)) and the rows' responses in a row
    // table; pass 2 adds the responses to the entering values and stores
    // the contributions over them.
    {
        const int I = wave, j = lane;
        const float ga = V(G_A)[j], gm = V(G_M)[j], gs = V(G_S)[j];
        // 0: m exits, 512: gcar exits, 1024: mcar exits, 1536 + 4 i: row
        // responses, 1792 + 4 I: block exit responses
        float* xch = Cm1;
        float m = 0.f, rp = 1.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int i = 8 * I + t;
            const float mi = readlane_f(gm, i);
            m = mi * m + (i == j ? 1.f : 0.f);
            cS_[i * LDC + j] = m;
            rp = mi * rp;
            if (j == 0) xch[1536 + 4 * i] = rp;
        }
        xch[64 * I + j] = m;
        const bool col = j < n;
        const float dml = -V(G_E)[j] * V(G_RZ2)[j];
        float dgc[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) dgc[t] = dGm[(8 * I + t) * LDC + j];
        float gc = 0.f, mc = 0.f;
        float PG = 1.f, QG = 0.f, QM = 1.f;   // response to carries (G, M) entering the block
#pragma unroll
        for (int t = 7; t >= 0; --t) {
            const int i = 8 * I + t;
            const bool act = col && i > j && i < n;
            const float ai = readlane_f(ga, i), si = readlane_f(gs, i), mi = readlane_f(gm, i);
            const float g = dgc[t] + gc;
            const float dmt = (i == n - 1 ? dml : 0.f) + mc + si * g;
            cA_[i * LDC + j] = g;
            cM_[i * LDC + j] = dmt;
            gc = act ? ai * g : gc;
            mc = act ? mi * dmt : mc;
            // the carries' response on row i: g += G PG, dmt += G (QG + beta_i
            // PG) + M QM (rows i < n carry it on; the same for every column
            // whose range covers the row)
            if (j == 0) {
                xch[1537 + 4 * i] = PG;
                xch[1538 + 4 * i] = QG;
                xch[1539 + 4 * i] = QM;
            }
            if (i < n) {
                QG = mi * (QG + si * PG);
                QM = mi * QM;
                PG = ai * PG;
            }
        }
        xch[512 + 64 * I + j] = gc;
        xch[1024 + 64 * I + j] = mc;
        if (j == 0) {
            xch[1792 + 4 * I] = PG;
            xch[1793 + 4 * I] = QG;
            xch[1794 + 4 * I] = QM;
        }
    }
    lds_barrier();
    {
        const int I = wave, j = lane;
        const float* xch = Cm1;
        // m entering the block (from the blocks above it in row order)
        float m0 = 0.f;
        for (int K = 0; K < I; ++K) m0 = xch[64 * K + j] + m0 * xch[1536 + 4 * (8 * K + 7)];
        // carries entering the block from row 8 I + 8 (the blocks below it
        // in row order, which the recursion runs first)
        float G = 0.f, M = 0.f;
        for (int K = 7; K > I; --K) {
            const float PGx = xch[1792 + 4 * K], QGx = xch[1793 + 4 * K], QMx = xch[1794 + 4 * K];
            const float Gn = xch[512 + 64 * K + j] + PGx * G;
            M = xch[1024 + 64 * K + j] + QGx * G + QMx * M;
            G = Gn;
        }
        const bool col = j < n;
        float mprev = m0;          // m_{i-1,j}
        float gnext = 0.f;         // g of row j + 1
        float mlast = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int i = 8 * I + t;
            const float4 r = *reinterpret_cast<const float4*>(xch + 1536 + 4 * i);
            const float si = V(G_S)[i];
            const float mcur = cS_[i * LDC + j] + m0 * r.x;
            const bool act = col && i > j && i < n;
            const float g = cA_[i * LDC + j] + G * r.y;
            const float dmt = cM_[i * LDC + j] + G * (r.z + si * r.y) + M * r.w;
            const float gprev = i > 0 ? Gm[(i - 1) * LDC + j] : 0.f;
            cA_[i * LDC + j] = act ? g * gprev : 0.f;
            cS_[i * LDC + j] = act ? g * mcur : 0.f;
            cM_[i * LDC + j] = act ? dmt * mprev : 0.f;
            gnext = i == j + 1 ? g : gnext;
            mlast = i == n - 1 ? mcur : mlast;
            mprev = mcur;
        }
        // gamma_{j,j} = beta_j: the carry entering row j is alpha_{j+1} g_{j+1}
        // (row j + 1 in this block) or, at the block's last row, G
        if (j >> 3 == I) {
            const float gin = (j & 7) == 7 ? G : (j + 1 < n ? V(G_A)[j + 1] * gnext : 0.f);
            cS_[j * LDC + j] = col ? dGm[j * LDC + j] + gin : 0.f;
        }
        if (col && (n - 1) >> 3 == I) V(G_DE)[j] += -mlast * V(G_RZ2)[j];
    }
    lds_barrier();
    for (int i = tid; i < CH; i += NT8) {
        float sa = 0.f, ss = 0.f, sm = 0.f;
        for (int j = 0; j < CH; ++j) {
            sa += cA_[i * LDC + j];
            ss += cS_[i * LDC + j];
            sm += cM_[i * LDC + j];
        }
        V(G_DA)[i] += sa;
        V(G_DS)[i] += ss;
        V(G_DM)[i] += sm;
    }
    lds_barrier();
    if (wave == 0) {
        const int i = lane;
        const bool in = i < n;
        const float anext = i + 1 < n ? V(G_A)[i + 1] : 0.f;
        const float mnext = i + 1 < n ? V(G_M)[i + 1] : 0.f;
        const float gb = bwd_suffix_affine(anext, in ? V(G_DB)[i] : 0.f, lane);
        const float bp = i > 0 ? V(G_B)[i - 1] : 0.f;
        float da = V(G_DA)[i] + gb * bp;
        const float ds = V(G_DS)[i] + gb * V(G_MB)[i];
        const float gmb0 = (in ? V(G_DMB)[i] : 0.f) + gb * V(G_S)[i];
        const float gab = bwd_suffix_affine(anext, in ? V(G_DAB)[i] : 0.f, lane);
        const float gmb = bwd_suffix_affine(mnext, in ? gmb0 : 0.f, lane);
        da += gab * (i > 0 ? V(G_AB)[i - 1] : 1.f);
        const float dm = V(G_DM)[i] + gmb * (i > 0 ? V(G_MB)[i - 1] : 1.f);
        if (in) {
            const size_t g = tok0 + (size_t)i * H;
            dalpha[g] = da;
            deta[g] = V(G_DE)[i];
            if (dmu) dmu[g] = dm;
            if (dbeta) dbeta[g] = ds;
        }
    }
}

// ---------------------------------------------------------------------------
// Reverse scan for bf16 I/O: the equations, column ownership and operand
// treatment of bwd_scan_kernel, in the layout of the forward's bf16 scan.
//  * Roles.  Eight wavefronts: 0..3 compute (wavefront w keeps columns
//    16 w .. 16 w + 15 of the workgroup's 64 of dS and dM for the whole
//    sequence), 4..7 stage chunk c - 1 with direct global-to-LDS loads (K, Q,
//    T, A, the workgroup's dO columns and the coefficient rows, all
//    row-major) while the compute wavefronts work on chunk c.  One barrier
//    per chunk hands the buffers over.
//  * Row order.  The state rows d and the chunk rows i of every accumulator
//    are in the forward scan's phys_row order, so a k-step fed from
//    accumulator tiles 2 s and 2 s + 1 covers the 8 contiguous rows
//    32 s + 8 g .. + 7.  Every operand whose k runs over chunk rows (A^T,
//    T^T, Q^T, K^T, and dO itself) is two transposing LDS reads of its
//    row-major tile; K's fragments for K dS' are 16-byte row reads.
//  * The exit-state gradients go to the workspace in bf16 as [d][v] rows:
//    each 16 x 16 tile is transposed on the matrix cores (a product with the
//    identity, exact on bf16 values) and lane groups g, g ^ 1 swap halves, so
//    that a lane stores 8 adjacent columns of one row.
//  * Workgroups are remapped so that the column tiles of a head run on one
//    XCD and read q, k, T and A through its L2 once.
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct BwdScanBf16Layout {
    using LK = TileLayout<DK * 2>;   // K, Q rows
    using LC = TileLayout<CH * 2>;   // T, A rows and the 64 dO columns
    static constexpr int TV = 64;    // value columns per workgroup
    static constexpr int OFF_Q = LK::BYTES;
    static constexpr int OFF_T = 2 * LK::BYTES;
    static constexpr int OFF_A = OFF_T + LC::BYTES;
    static constexpr int OFF_G = OFF_A + LC::BYTES;
    static constexpr int OFF_VEC = OFF_G + LC::BYTES;
    static constexpr int BUF_BYTES = OFF_VEC + 6 * CH * 4;
    // bytes from row x to row 32 s + x (s = 1), and from row x to row x + 4
    // for the rows 8 g + (0..3) the transposing reads start at
    static constexpr int KSTEP = 32 * (DK * 2) + (32 / LK::G) * LK::PAD;
    static constexpr int CSTEP = 32 * (CH * 2) + (32 / LC::G) * LC::PAD;
    static constexpr int KHALF = 4 * (DK * 2) + (LK::G == 4 ? LK::PAD : 0);
    static constexpr int CHALF = 4 * (CH * 2) + (LC::G == 4 ? LC::PAD : 0);
};

__device__ __forceinline__ bf16x4 bwd_to_bf4(const f32x4& x)
{
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
    return __builtin_bit_cast(bf16x4, u32x2_t{bwd_pack_bf16(x[0], x[1]), bwd_pack_bf16(x[2], x[3])});
}
// x as a bf16 head and a bf16 remainder (x - head), both rounded to nearest
__device__ __forceinline__ void bwd_split8(const float* x, bf16x8& hd, bf16x8& rs)
{
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
    u32x4_t h, r;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        h[u] = bwd_pack_bf16(x[2 * u], x[2 * u + 1]);
        const float h0 = __uint_as_float(h[u] << 16);
        const float h1 = __uint_as_float(h[u] & 0xffff0000u);
        r[u] = bwd_pack_bf16(x[2 * u] - h0, x[2 * u + 1] - h1);
    }
    hd = __builtin_bit_cast(bf16x8, h);
    rs = __builtin_bit_cast(bf16x8, r);
}

template <int DK, int DV>
__global__ __launch_bounds__(NT8) void bwd_scan_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ dO,
    const __bf16* __restrict__ Tw, const __bf16* __restrict__ Aw, const float* __restrict__ Vw,
    const float* dST, const float* dMT, __bf16* __restrict__ Hd, float* __restrict__ dv,
    float* dS0, float* dM0, int T, int H, int NC, int xcd_groups)
{
    using MB = Mma<__bf16>;
    using L = BwdScanBf16Layout<DK, DV>;
    using LK = typename L::LK;
    using LC = typename L::LC;
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
    constexpr int TV = L::TV;
    constexpr int NTILE = DV / TV;
    constexpr int RT = DK / 16;   // state row tiles
    constexpr int SK = DK / 32;   // k-steps over d
    constexpr int SC = CH / 32;   // k-steps over the chunk rows
    static_assert(DV % TV == 0 && RT % 2 == 0, "tiles");

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
        const unsigned g_stride = (unsigned)(H * DV);
        const unsigned g_lane = LC::lane_offset(g_stride, lane);
        auto stage = [&](int c, int bi) {
            const int n = min(CH, T - c * CH);
            const size_t tok0 = ((size_t)b * T + c * CH) * H + h;
            const size_t chn = (size_t)bh * NC + c;
            char* B = buf[bi];
            LK::load(B, k + tok0 * DK, kq_stride, kq_lane, n, hw, lane);
            LK::load(B + L::OFF_Q, q + tok0 * DK, kq_stride, kq_lane, n, hw, lane);
            LC::load(B + L::OFF_T, Tw + chn * CH * CH, CH, c_lane, CH, hw, lane);
            LC::load(B + L::OFF_A, Aw + chn * CH * CH, CH, c_lane, CH, hw, lane);
            // this tile's 64 columns of dO (rows >= n read row n - 1; A's and
            // the coefficient rows' zero rows >= n keep them out of every sum)
            LC::load(B + L::OFF_G, dO + tok0 * DV + tile * TV, g_stride, g_lane, n, hw, lane);
            // coefficient vectors: 6 x 64 floats = 96 pieces of 16 bytes
            if (hw == 0 || (hw == 1 && lane < 32))
                direct_load16(Vw + chn * NVEC * CH + 4 * (64 * hw + lane),
                              B + L::OFF_VEC + 1024 * hw);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        };
        stage(NC - 1, (NC - 1) & 1);
        lds_barrier();
        for (int c = NC - 1; c >= 0; --c) {
            if (c > 0) stage(c - 1, (c - 1) & 1);
            lds_barrier();
        }
        return;
    }

    // ---------------- compute wavefronts ----------------
    const int wcol = tile * TV + 16 * wave;   // first column of this wavefront in the head
    const int col = wcol + l16;
    // dS, dM: slot (rt, lg, r) is state row phys_row(16 rt + 4 lg + r)
    f32x4 Sa[RT], Ma[RT];
    const size_t sbase = (size_t)bh * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const size_t x = sbase + (size_t)phys_row(16 * rt + 4 * lg + r) * DV + col;
            Sa[rt][r] = dST ? dST[x] : 0.f;
            Ma[rt][r] = dMT ? dMT[x] : 0.f;
        }

    // per-lane LDS offsets (bytes), the same every chunk
    //  kq_base[x]: K row phys_row(16 x + l16), 16-byte chunk lg (the A
    //    fragments of K dS'; step s is 64 s bytes further)
    //  ktr: transposing reads of K or Q -- lane 4 j + m of group lg reads row
    //    8 lg + 4 hf + j (+ 32 s), columns phys_row(16 rt + 4 m) .. + 3, so
    //    lane l16 gets column phys_row(16 rt + l16) of those rows: the A
    //    fragment of K^T or Q^T for state tile rt (+ 64 (rt >> 1) + 8 (rt & 1)
    //    bytes, + KHALF for hf = 1, + KSTEP per step)
    //  ctr: the same over a 64-column tile (T, A), columns phys_row(16 x + 4 m)
    //  g_off: dO rows 8 lg + 4 hf + j, columns 16 w + 4 m .. + 3 of the 64:
    //    lane l16 gets column 16 w + l16, the B fragment of dO
    int kq_base[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) kq_base[x] = LK::chunk(phys_row(16 * x + l16), lg);
    const int ktr = LK::chunk(8 * lg + (l16 >> 2), l16 & 3);
    const int ctr = LC::chunk(8 * lg + (l16 >> 2), l16 & 3);
    const int c4 = 16 * wave + 4 * (l16 & 3);
    const int g_off = L::OFF_G + LC::chunk(8 * lg + (l16 >> 2), c4 >> 3) + 2 * (c4 & 7);
    auto kt_at = [&](const char* base, int rt, int s) {
        const int o = ktr + 64 * (rt >> 1) + 8 * (rt & 1) + s * L::KSTEP;
        return bwd_cat8(lds_read_tr4(base + o), lds_read_tr4(base + o + L::KHALF));
    };
    auto ct_at = [&](const char* base, int x, int s) {
        const int o = ctr + 64 * (x >> 1) + 8 * (x & 1) + s * L::CSTEP;
        return bwd_cat8(lds_read_tr4(base + o), lds_read_tr4(base + o + L::CHALF));
    };
    // the 16 x 16 identity as a B fragment of mma16: B[4 lg + j][l16] = (4 lg + j == l16)
    bf16x4 eye;
#pragma unroll
    for (int j = 0; j < 4; ++j) eye[j] = static_cast<__bf16>(4 * lg + j == l16 ? 1.f : 0.f);
    const unsigned vstride = (unsigned)(H * DV);

    // The exit-state gradients go to the workspace in bf16, [d][v] rows: each
    // 16 x 16 tile is transposed by a product with the identity, after which
    // lane (l16, g) holds row phys_row(16 rt + l16), columns 4 g .. + 3; lane
    // groups g and g ^ 1 then swap halves of tiles 2 p and 2 p + 1
    // (permlane16_swap exchanges group 1 of its first operand with group 0 of
    // its second, and group 3 with group 2), so that each lane holds columns
    // 8 (g >> 1) .. + 7 of row phys_row(16 (2 p + (g & 1)) + l16).
    auto store_pair = [&](__bf16* hd, int p, const bf16x4& t0, const bf16x4& t1) {
        u32x2_t ua = __builtin_bit_cast(u32x2_t, bwd_to_bf4(mma16(t0, eye, zero4())));
        u32x2_t ub = __builtin_bit_cast(u32x2_t, bwd_to_bf4(mma16(t1, eye, zero4())));
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const auto r = __builtin_amdgcn_permlane16_swap(ua[d], ub[d], false, false);
            ua[d] = r[0];
            ub[d] = r[1];
        }
        const int row = phys_row(16 * (2 * p + (lg & 1)) + l16);
        *reinterpret_cast<u32x4_t*>(hd + row * DV) = u32x4_t{ua[0], ua[1], ub[0], ub[1]};
    };

    // chunk c's exit-state gradients dS', dM' (the current dS, dM), as the
    // bf16 values K dS' and K dM' use, to the workspace
    auto store_exit = [&](int c) {
        __bf16* const hd = Hd + ((size_t)bh * NC + c) * 2 * DK * DV + wcol + 8 * (lg >> 1);
#pragma unroll
        for (int p = 0; p < RT / 2; ++p) {
            store_pair(hd, p, bwd_to_bf4(Sa[2 * p]), bwd_to_bf4(Sa[2 * p + 1]));
            store_pair(hd + (size_t)DK * DV, p, bwd_to_bf4(Ma[2 * p]), bwd_to_bf4(Ma[2 * p + 1]));
        }
    };

    store_exit(NC - 1);
    lds_barrier();   // chunk NC - 1 staged
    for (int c = NC - 1; c >= 0; --c) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const char* Kb = buf[c & 1];
        const char* Qb = Kb + L::OFF_Q;
        const char* Tb = Kb + L::OFF_T;
        const char* Ab = Kb + L::OFF_A;
        const float* vec = reinterpret_cast<const float*>(Kb + L::OFF_VEC);

        // K dS', K dM': rows phys_row(16 ct + 4 lg + r) of the chunk
        f32x4 xs[4], xm[4];
        auto k_ds = [&]() {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) xs[ct] = xm[ct] = zero4();
#pragma unroll
            for (int s = 0; s < SK; ++s) {
                const bf16x8 bS = bwd_cat8(bwd_to_bf4(Sa[2 * s]), bwd_to_bf4(Sa[2 * s + 1]));
                const bf16x8 bM = bwd_cat8(bwd_to_bf4(Ma[2 * s]), bwd_to_bf4(Ma[2 * s + 1]));
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const bf16x8 aK = *reinterpret_cast<const bf16x8*>(Kb + kq_base[ct] + 64 * s);
                    xs[ct] = MB::mma(aK, bS, xs[ct]);
                    xm[ct] = MB::mma(aK, bM, xm[ct]);
                }
            }
        };
        // the state gradients' own carry: dS <- abar_n dS', dM <- mubar_n dM' - b_n dS'
        auto decay = [&]() {
            const float abn = vec[V_SCAL * CH + 0];
            const float bn = vec[V_SCAL * CH + 1];
            const float mbn = vec[V_SCAL * CH + 2];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 so = Sa[rt];
                Sa[rt] = abn * so;
                Ma[rt] = mbn * Ma[rt] - bn * so;
            }
        };
        // dO fragments: rows 32 s + 8 lg + (0..7), column col
        bf16x8 gf[SC];
#pragma unroll
        for (int s = 0; s < SC; ++s)
            gf[s] = bwd_cat8(lds_read_tr4(Kb + g_off + s * L::CSTEP),
                             lds_read_tr4(Kb + g_off + s * L::CSTEP + L::CHALF));
        // dS += X^T Diag(su u) Y, dM += X^T Diag(sw w) Y over the chunk rows,
        // for X = Q or K (transposing reads) and Y given by y(s, j) (rows
        // 32 s + 8 lg + j); the scaled rows as head and remainder
        auto carry = [&](const char* Xb, const float* u, float su, const float* w, float sw,
                         auto y, int s0, int s1) {
#pragma unroll
            for (int s = s0; s < s1; ++s) {
                float xs8[8], xm8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float yv = y(s, j);
                    xs8[j] = su * u[32 * s + 8 * lg + j] * yv;
                    xm8[j] = sw * w[32 * s + 8 * lg + j] * yv;
                }
                bf16x8 sh, sr, mh, mr;
                bwd_split8(xs8, sh, sr);
                bwd_split8(xm8, mh, mr);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const bf16x8 aX = kt_at(Xb, rt, s);
                    Sa[rt] = MB::mma(aX, sh, Sa[rt]);
                    Sa[rt] = MB::mma(aX, sr, Sa[rt]);
                    Ma[rt] = MB::mma(aX, mh, Ma[rt]);
                    Ma[rt] = MB::mma(aX, mr, Ma[rt]);
                }
            }
        };
        // dVt = Diag(ws) K dS' - Diag(wm) K dM' + A^T dO, then dR = T^T dVt (dVt
        // as head and remainder), written as dv
        f32x4 dR[4], dVt[4];
        auto dvt = [&]() {
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int p0 = phys_row(16 * it + 4 * lg);
                const f32x4 ws = *reinterpret_cast<const f32x4*>(vec + V_WS * CH + p0);
                const f32x4 wm = *reinterpret_cast<const f32x4*>(vec + V_WM * CH + p0);
                dVt[it] = ws * xs[it] - wm * xm[it];
            }
#pragma unroll
            for (int s = 0; s < SC; ++s)
#pragma unroll
                for (int it = 0; it < 4; ++it) dVt[it] = MB::mma(ct_at(Ab, it, s), gf[s], dVt[it]);
        };
        auto dr = [&]() {
#pragma unroll
            for (int it = 0; it < 4; ++it) dR[it] = zero4();
#pragma unroll
            for (int s = 0; s < SC; ++s) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[j] = dVt[2 * s][j];
                    x[4 + j] = dVt[2 * s + 1][j];
                }
                bf16x8 vh, vr;
                bwd_split8(x, vh, vr);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const bf16x8 aT = ct_at(Tb, it, s);
                    dR[it] = MB::mma(aT, vh, dR[it]);
                    dR[it] = MB::mma(aT, vr, dR[it]);
                }
            }
            // a wave-uniform base and 32-bit lane offsets; no row tests in a
            // full chunk
            float* dvb = dv + (((size_t)b * T + t0) * H + h) * DV + wcol;
            if (n == CH) {
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        dvb[(unsigned)phys_row(16 * it + 4 * lg + r) * vstride + (unsigned)l16] =
                            dR[it][r];
            } else {
#pragma unroll
                for (int it = 0; it < 4; ++it)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = phys_row(16 * it + 4 * lg + r);
                        if (i < n) dvb[(unsigned)i * vstride + (unsigned)l16] = dR[it][r];
                    }
            }
        };

        // dS += Q^T Diag(abar) dO - K^T Diag(abar) dR,
        // dM += -Q^T Diag(b) dO + K^T Diag(ab1) dR
        auto carry_q = [&](int s0, int s1) {
            carry(Qb, vec + V_ABAR * CH, 1.f, vec + V_B * CH, -1.f,
                  [&](int s, int j) { return static_cast<float>(gf[s][j]); }, s0, s1);
        };
        auto carry_k = [&](int s0, int s1) {
            carry(Kb, vec + V_ABAR * CH, -1.f, vec + V_AB1 * CH, 1.f,
                  [&](int s, int j) { return j < 4 ? dR[2 * s][j] : dR[2 * s + 1][j - 4]; }, s0,
                  s1);
        };
        k_ds();
        decay();
        carry_q(0, SC);
        dvt();
        dr();
        carry_k(0, SC);
        if (c > 0) store_exit(c - 1);
        lds_barrier();   // this chunk's buffer is free and the previous chunk is staged
    }

    // (the lane's row group through an empty asm: addresses formed here, not
    // kept in registers across the loop)
    int lgx = lg;
    asm volatile("" : "+v"(lgx));
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const size_t x = sbase + (size_t)phys_row(16 * rt + 4 * lgx + r) * DV + col;
            if (dS0) dS0[x] = Sa[rt][r];
            if (dM0) dM0[x] = Ma[rt][r];
        }
}

// ---------------------------------------------------------------------------
// Forward re-scan for bf16 I/O: the equations and operand treatment of
// bwd_rescan_kernel (S and M rounded to bf16 in K S, K M; R and the
// weight-scaled rows of Vt split into a bf16 head and remainder), in the
// layout of the reverse scan above: four compute wavefronts with 16 state
// columns each, four staging wavefronts loading chunk c + 1 (K, the
// workgroup's columns of v or of the saved Vt, T unless Vt was saved, the
// coefficient rows) with direct global-to-LDS loads, one barrier per chunk.
// Each chunk's entry state goes to the workspace in bf16, [d][v] rows, as
// the reverse scan stores the exit-state gradients; without saved residuals
// the chunk's Vt goes there too, in fp32.
// ---------------------------------------------------------------------------
template <int DK, int DV, bool SAVED>
struct BwdRescanBf16Layout {
    using LK = TileLayout<DK * 2>;   // K rows
    using LC = TileLayout<CH * 2>;   // T rows and the 64 columns of v (or Vt)
    static constexpr int TV = 64;
    static constexpr int OFF_V = LK::BYTES;
    static constexpr int OFF_T = OFF_V + LC::BYTES;
    static constexpr int OFF_VEC = OFF_T + (SAVED ? 0 : LC::BYTES);
    static constexpr int BUF_BYTES = OFF_VEC + 6 * CH * 4;
    static constexpr int KSTEP = 32 * (DK * 2) + (32 / LK::G) * LK::PAD;
    static constexpr int CSTEP = 32 * (CH * 2) + (32 / LC::G) * LC::PAD;
    static constexpr int KHALF = 4 * (DK * 2) + (LK::G == 4 ? LK::PAD : 0);
    static constexpr int CHALF = 4 * (CH * 2) + (LC::G == 4 ? LC::PAD : 0);
};

template <int DK, int DV, bool SAVED>
__global__ __launch_bounds__(NT8) void bwd_rescan_bf16_kernel(
    const __bf16* __restrict__ k, const __bf16* __restrict__ v, const __bf16* __restrict__ Tw,
    const float* __restrict__ Vw, const float* S0, const float* M0, __bf16* __restrict__ Hs,
    float* __restrict__ Vts, int T, int H, int NC, int xcd_groups)
{
    using MB = Mma<__bf16>;
    using L = BwdRescanBf16Layout<DK, DV, SAVED>;
    using LK = typename L::LK;
    using LC = typename L::LC;
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
    constexpr int TV = L::TV;
    constexpr int NTILE = DV / TV;
    constexpr int RT = DK / 16;   // state row tiles
    constexpr int SK = DK / 32;   // k-steps over d
    constexpr int SC = CH / 32;   // k-steps over the chunk rows
    static_assert(DV % TV == 0 && RT % 2 == 0, "tiles");

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
        const unsigned k_stride = (unsigned)(H * DK);
        const unsigned k_lane = LK::lane_offset(k_stride, lane);
        const unsigned c_lane = LC::lane_offset(CH, lane);
        const unsigned v_stride = (unsigned)(H * DV);
        const unsigned v_lane = LC::lane_offset(v_stride, lane);
        auto stage = [&](int c, int bi) {
            const int n = min(CH, T - c * CH);
            const size_t tok0 = ((size_t)b * T + c * CH) * H + h;
            const size_t chn = (size_t)bh * NC + c;
            char* B = buf[bi];
            LK::load(B, k + tok0 * DK, k_stride, k_lane, n, hw, lane);
            // rows >= n read row n - 1; their weights (and R's rows, through
            // T's identity rows) keep them out of the update
            LC::load(B + L::OFF_V, v + tok0 * DV + tile * TV, v_stride, v_lane, n, hw, lane);
            if constexpr (!SAVED) LC::load(B + L::OFF_T, Tw + chn * CH * CH, CH, c_lane, CH, hw, lane);
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
    const int wcol = tile * TV + 16 * wave;   // first column of this wavefront in the head
    const int col = wcol + l16;
    // S, M: slot (rt, lg, r) is state row phys_row(16 rt + 4 lg + r)
    f32x4 Sa[RT], Ma[RT];
    const size_t sbase = (size_t)bh * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const size_t x = sbase + (size_t)phys_row(16 * rt + 4 * lg + r) * DV + col;
            Sa[rt][r] = S0 ? S0[x] : 0.f;
            Ma[rt][r] = M0 ? M0[x] : 0.f;
        }

    // per-lane LDS offsets (bytes), as in the reverse scan:
    //  kq_base[x]: K row phys_row(16 x + l16), 16-byte chunk lg (K S, K M)
    //  c_base[x]: T row phys_row(16 x + l16), 16-byte chunk lg (T R)
    //  ktr: transposing reads of K (the A fragments of K^T)
    //  v_r[x]: v rows phys_row(16 x + 4 lg) + j, columns 16 w + 4 m .. + 3:
    //    lane l16 gets column col of those four rows, R's layout
    //  v_t: the same tile's rows 8 lg + 4 hf + j (+ 32 s): the B fragment of
    //    a saved Vt
    int kq_base[4], c_base[4], v_r[4];
    const int c4 = 16 * wave + 4 * (l16 & 3);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int r = phys_row(16 * x + l16);
        kq_base[x] = LK::chunk(r, lg);
        c_base[x] = L::OFF_T + LC::chunk(r, lg);
        v_r[x] = L::OFF_V + LC::chunk(phys_row(16 * x + 4 * lg) + (l16 >> 2), c4 >> 3) + 2 * (c4 & 7);
    }
    const int ktr = LK::chunk(8 * lg + (l16 >> 2), l16 & 3);
    const int v_t = L::OFF_V + LC::chunk(8 * lg + (l16 >> 2), c4 >> 3) + 2 * (c4 & 7);
    auto kt_at = [&](const char* base, int rt, int s) {
        const int o = ktr + 64 * (rt >> 1) + 8 * (rt & 1) + s * L::KSTEP;
        return bwd_cat8(lds_read_tr4(base + o), lds_read_tr4(base + o + L::KHALF));
    };
    bf16x4 eye;
#pragma unroll
    for (int j = 0; j < 4; ++j) eye[j] = static_cast<__bf16>(4 * lg + j == l16 ? 1.f : 0.f);

    // chunk c's entry state (the current S, M) to the workspace in bf16, [d][v]
    // rows, transposed per 16 x 16 tile on the matrix cores as in the reverse scan
    auto store_pair = [&](__bf16* hs, int p, const bf16x4& t0, const bf16x4& t1) {
        u32x2_t ua = __builtin_bit_cast(u32x2_t, bwd_to_bf4(mma16(t0, eye, zero4())));
        u32x2_t ub = __builtin_bit_cast(u32x2_t, bwd_to_bf4(mma16(t1, eye, zero4())));
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const auto r = __builtin_amdgcn_permlane16_swap(ua[d], ub[d], false, false);
            ua[d] = r[0];
            ub[d] = r[1];
        }
        const int row = phys_row(16 * (2 * p + (lg & 1)) + l16);
        *reinterpret_cast<u32x4_t*>(hs + row * DV) = u32x4_t{ua[0], ua[1], ub[0], ub[1]};
    };
    auto store_entry = [&](int c) {
        __bf16* const hs = Hs + ((size_t)bh * NC + c) * 2 * DK * DV + wcol + 8 * (lg >> 1);
#pragma unroll
        for (int p = 0; p < RT / 2; ++p) {
            store_pair(hs, p, bwd_to_bf4(Sa[2 * p]), bwd_to_bf4(Sa[2 * p + 1]));
            store_pair(hs + (size_t)DK * DV, p, bwd_to_bf4(Ma[2 * p]), bwd_to_bf4(Ma[2 * p + 1]));
        }
    };

    store_entry(0);
    lds_barrier();   // chunk 0 staged
    for (int c = 0; c < NC; ++c) {
        const char* Kb = buf[c & 1];
        const float* vec = reinterpret_cast<const float*>(Kb + L::OFF_VEC);

        // Vt of this chunk: rows 32 s + 8 lg + (0..7) of column col as the
        // update's B operands (weighted and split below)
        f32x4 Vt[4];
        if constexpr (!SAVED) {
            // X = K [S | M], R = V - Diag(abar) K S + Diag(ab1) K M, Vt = T R (R
            // as head and remainder); rows phys_row(16 x + 4 lg + r)
            f32x4 xs[4], xm[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) xs[ct] = xm[ct] = zero4();
#pragma unroll
            for (int s = 0; s < SK; ++s) {
                const bf16x8 bS = bwd_cat8(bwd_to_bf4(Sa[2 * s]), bwd_to_bf4(Sa[2 * s + 1]));
                const bf16x8 bM = bwd_cat8(bwd_to_bf4(Ma[2 * s]), bwd_to_bf4(Ma[2 * s + 1]));
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const bf16x8 aK = *reinterpret_cast<const bf16x8*>(Kb + kq_base[ct] + 64 * s);
                    xs[ct] = MB::mma(aK, bS, xs[ct]);
                    xm[ct] = MB::mma(aK, bM, xm[ct]);
                }
            }
            f32x4 R[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int p0 = phys_row(16 * ct + 4 * lg);
                const f32x4 ab = *reinterpret_cast<const f32x4*>(vec + V_ABAR * CH + p0);
                const f32x4 ab1 = *reinterpret_cast<const f32x4*>(vec + V_AB1 * CH + p0);
                const bf16x4 vv = lds_read_tr4(Kb + v_r[ct]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    R[ct][r] = static_cast<float>(vv[r]) - ab[r] * xs[ct][r] + ab1[r] * xm[ct][r];
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) Vt[it] = zero4();
#pragma unroll
            for (int s = 0; s < SC; ++s) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[j] = R[2 * s][j];
                    x[4 + j] = R[2 * s + 1][j];
                }
                bf16x8 rh, rr;
                bwd_split8(x, rh, rr);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const bf16x8 aT = *reinterpret_cast<const bf16x8*>(Kb + c_base[it] + 64 * s);
                    Vt[it] = MB::mma(aT, rh, Vt[it]);
                    Vt[it] = MB::mma(aT, rr, Vt[it]);
                }
            }
            // to the workspace in fp32, [chunk row][v]
            float* vb = Vts + ((size_t)bh * NC + c) * CH * DV + wcol;
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vb[(unsigned)phys_row(16 * it + 4 * lg + r) * DV + (unsigned)l16] = Vt[it][r];
        }

        // S' = abar_n S - b_n M + K^T Diag(ws) Vt,  M' = mubar_n M - K^T Diag(wm) Vt
        {
            const float abn = vec[V_SCAL * CH + 0];
            const float bn = vec[V_SCAL * CH + 1];
            const float mbn = vec[V_SCAL * CH + 2];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                Sa[rt] = abn * Sa[rt] - bn * Ma[rt];
                Ma[rt] = mbn * Ma[rt];
            }
        }
#pragma unroll
        for (int s = 0; s < SC; ++s) {
            float y[8];
            if constexpr (SAVED) {
                const bf16x8 g = bwd_cat8(lds_read_tr4(Kb + v_t + s * L::CSTEP),
                                          lds_read_tr4(Kb + v_t + s * L::CSTEP + L::CHALF));
#pragma unroll
                for (int j = 0; j < 8; ++j) y[j] = static_cast<float>(g[j]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    y[j] = Vt[2 * s][j];
                    y[4 + j] = Vt[2 * s + 1][j];
                }
            }
            const float* ws = vec + V_WS * CH + 32 * s + 8 * lg;
            const float* wm = vec + V_WM * CH + 32 * s + 8 * lg;
            float xs8[8], xm8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                xs8[j] = ws[j] * y[j];
                xm8[j] = -(wm[j] * y[j]);
            }
            bf16x8 sh, sr, mh, mr;
            bwd_split8(xs8, sh, sr);
            bwd_split8(xm8, mh, mr);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const bf16x8 aK = kt_at(Kb, rt, s);
                Sa[rt] = MB::mma(aK, sh, Sa[rt]);
                Sa[rt] = MB::mma(aK, sr, Sa[rt]);
                Ma[rt] = MB::mma(aK, mh, Ma[rt]);
                Ma[rt] = MB::mma(aK, mr, Ma[rt]);
            }
        }
        if (c + 1 < NC) store_entry(c + 1);
        lds_barrier();   // this chunk's buffer is free and the next one is staged
    }
}

}  // namespace
}  // namespace mdn

namespace mdn {

size_t chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, bool bf16)
{
    const size_t NC = ((size_t)T + CH - 1) / CH;
    const size_t nchunks = (size_t)B * H * NC;
    const size_t prep = nchunks * (2 * CH * CH * (bf16 ? 2 : 4) + NVEC * CH * 4);
    // state pairs in the I/O type, residuals in fp32
    return prep + nchunks * (4 * (size_t)Dk * Dv * (bf16 ? 2 : 4) + (size_t)CH * Dv * 4);
}

template <typename E, int DK, int DV>
static hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const float* alpha,
                               const float* mu, const float* eta, const float* beta,
                               const float* S0, const float* M0, const void* dO,
                               const float* dST, const float* dMT, const void* Vsaved, float* dq,
                               float* dk,
                               float* dv, float* dalpha, float* dmu, float* deta, float* dbeta,
                               float* dS0, float* dM0, int B, int T, int H, void* workspace,
                               hipStream_t stream)
{
    const int NC = (T + CH - 1) / CH;
    const size_t nchunks = (size_t)B * H * NC;
    char* p = static_cast<char*>(workspace);
    E* Tw = reinterpret_cast<E*>(p);
    p += nchunks * CH * CH * sizeof(E);
    E* Aw = reinterpret_cast<E*>(p);
    p += nchunks * CH * CH * sizeof(E);
    float* Vw = reinterpret_cast<float*>(p);
    p += nchunks * NVEC * CH * sizeof(float);
    E* Hs = reinterpret_cast<E*>(p);
    p += nchunks * 2 * DK * DV * sizeof(E);
    E* Hd = reinterpret_cast<E*>(p);
    p += nchunks * 2 * DK * DV * sizeof(E);
    float* Vts = reinterpret_cast<float*>(p);

    hipError_t err = launch_chunk_prepare(q, k, alpha, mu, eta, beta, B, T, H, DK,
                                          sizeof(E) == 2, workspace, stream);
    if (err != hipSuccess) return err;
    const unsigned nblk = (unsigned)((size_t)B * H * (DV / 64));
    if constexpr (sizeof(E) == 2) {
        // column tiles of a head on one XCD (consecutive ids after the remap)
        const int xcd_groups = nblk % 8 == 0 ? (int)(nblk / 8) : 0;
        hipLaunchKernelGGL((bwd_scan_bf16_kernel<DK, DV>), dim3(nblk), dim3(NT8), 0, stream,
                           static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                           static_cast<const __bf16*>(dO), Tw, Aw, Vw, dST, dMT, Hd, dv, dS0,
                           dM0, T, H, NC, xcd_groups);
    } else {
        hipLaunchKernelGGL((bwd_scan_kernel<E, DK, DV>), dim3(nblk), dim3(NT), 0, stream,
                           static_cast<const E*>(q), static_cast<const E*>(k),
                           static_cast<const E*>(dO), Tw, Aw, Vw, dST, dMT, Hd, dv, dS0, dM0, T,
                           H, NC);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if constexpr (sizeof(E) == 2) {
        const int xcd_groups = nblk % 8 == 0 ? (int)(nblk / 8) : 0;
        if (Vsaved)
            hipLaunchKernelGGL((bwd_rescan_bf16_kernel<DK, DV, true>), dim3(nblk), dim3(NT8), 0,
                               stream, static_cast<const __bf16*>(k),
                               static_cast<const __bf16*>(Vsaved), Tw, Vw, S0, M0, Hs, Vts, T, H,
                               NC, xcd_groups);
        else
            hipLaunchKernelGGL((bwd_rescan_bf16_kernel<DK, DV, false>), dim3(nblk), dim3(NT8), 0,
                               stream, static_cast<const __bf16*>(k),
                               static_cast<const __bf16*>(v), Tw, Vw, S0, M0, Hs, Vts, T, H, NC,
                               xcd_groups);
    } else if (Vsaved) {
        hipLaunchKernelGGL((bwd_rescan_kernel<E, DK, DV, true>), dim3(nblk), dim3(NT), 0, stream,
                           static_cast<const E*>(k), static_cast<const E*>(Vsaved), Tw, Vw, S0,
                           M0, Hs, Vts, T, H, NC);
    } else {
        hipLaunchKernelGGL((bwd_rescan_kernel<E, DK, DV, false>), dim3(nblk), dim3(NT), 0,
                           stream, static_cast<const E*>(k), static_cast<const E*>(v), Tw, Vw,
                           S0, M0, Hs, Vts, T, H, NC);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if constexpr (sizeof(E) == 2)
        hipLaunchKernelGGL((Vsaved ? bwd_grad_bf16_kernel<DK, DV, true>
                                   : bwd_grad_bf16_kernel<DK, DV, false>),
                           dim3((unsigned)nchunks), dim3(NT8), 0,
                           stream, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                           static_cast<const __bf16*>(dO), dv, Vts,
                           static_cast<const __bf16*>(Vsaved), Hs, Hd, alpha, mu, eta, beta, dq,
                           dk, dalpha, dmu, deta, dbeta, S0, M0, dST, dMT, T, H, NC);
    else
        hipLaunchKernelGGL((bwd_grad_kernel<E, DK, DV>), dim3((unsigned)nchunks), dim3(NT), 0,
                           stream, static_cast<const E*>(q), static_cast<const E*>(k),
                           static_cast<const E*>(dO), dv, Vts, static_cast<const E*>(Vsaved), Hs,
                           Hd, alpha, mu, eta, beta, dq, dk, dalpha, dmu, deta, dbeta, T, H, NC);
    return hipGetLastError();
}

hipError_t launch_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                            const float* mu, const float* eta, const float* beta, const float* S0,
                            const float* M0, const void* dO, const float* dST, const float* dMT,
                            const void* Vsaved, float* dq, float* dk, float* dv, float* dalpha,
                            float* dmu, float* deta, float* dbeta, float* dS0, float* dM0, int B,
                            int T, int H, int Dk, int Dv, bool bf16, void* workspace,
                            hipStream_t stream)
{
#define MDN_BWD(E, DK, DV)                                                                        \
    if (Dk == DK && Dv == DV)                                                                     \
        return launch_bwd_t<E, DK, DV>(q, k, v, alpha, mu, eta, beta, S0, M0, dO, dST, dMT,       \
                                       Vsaved, dq,                                                \
                                       dk, dv, dalpha, dmu, deta, dbeta, dS0, dM0, B, T, H,       \
                                       workspace, stream);
    if (bf16) {
        MDN_BWD(__bf16, 64, 64) MDN_BWD(__bf16, 64, 128)
        MDN_BWD(__bf16, 128, 64) MDN_BWD(__bf16, 128, 128)
    } else {
        MDN_BWD(float, 64, 64) MDN_BWD(float, 64, 128)
        MDN_BWD(float, 128, 64) MDN_BWD(float, 128, 128)
    }
#undef MDN_BWD
    return hipErrorInvalidValue;
}

}  // namespace mdn
