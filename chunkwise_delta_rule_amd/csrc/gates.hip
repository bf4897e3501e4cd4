// gates.hip -- MDN's coupled gate parameterisation on gfx950.
//
// From per-token, per-head logits (the caller's projections of the layer
// input) to the four gates of the recurrence, as in "MDN: Parallelizing
// Stepwise Momentum for Delta Linear Attention" (slides), frame "Coupled gates
// restrict the spectral region" (the paper's Sec. 3.3); the reading notes on
// the same paper, Sec. 2.8, give the same equations:
//     eta   = 1 + tanh(z_eta / tau)                  in (0, 2)
//     theta = arctan(s eta),  alpha_max = cos^2 theta,  beta_max = sin^2 theta
//     log alpha = f(z_alpha) + log alpha_max
//     beta      = sigmoid(z_beta) beta_max
//     log mu    = max(f(z_mu), log_mu_min)
// with f(z) = -a softplus(z + b), so that alpha + beta <= 1 for a >= 0.
//
// How it is evaluated (each form equal to the one above in real arithmetic):
//   - alpha_max and beta_max from cos^2(arctan x) = 1 / (1 + x^2) and
//     sin^2(arctan x) = x^2 / (1 + x^2): no trigonometric function;
//   - eta = 2 / (1 + e^(-2 z_eta / tau)), which keeps its relative precision
//     where eta approaches 0 (1 + tanh cancels there);
//   - everything in base 2 on the hardware's exp2, log2 and reciprocal
//     (v_exp_f32, v_log_f32, v_rcp_f32): with L = log2 e and
//     sp2(y) = max(y, 0) + log2(1 + 2^-|y|) = softplus(y / L) L,
//         alpha = alpha_max 2^(-a sp2((z_alpha + b) L))
//         mu    = 2^max(-a sp2((z_mu + b) L), log_mu_min L)
//         beta  = beta_max / (1 + 2^(-z_beta L))
//     All of them stay finite for any finite logit.  Each result carries
//     about |ln result| + a few ulps of relative error: the rounding of the
//     exponent's argument, scaled by the exponential.
//
// The transform is elementwise and bound by HBM traffic: 16 bytes read and
// 16 bytes written per token and head.  Each thread handles V consecutive
// elements with 4V-byte accesses, in a grid-stride loop.
#include <hip/hip_runtime.h>

namespace mdn {

namespace {

constexpr float LOG2E = 1.4426950408889634f;

struct GateConsts {
    float eta_scale;    // -2 L / tau
    float s;
    float a;
    float bL;           // b L
    float floorL;       // log_mu_min L
};

template <int V>
using fvec = float __attribute__((ext_vector_type(V)));

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(y / L) L, for y already in base-2 units
__device__ __forceinline__ float sp2(float y) { return fmaxf(y, 0.f) + lg2(1.f + ex2(-fabsf(y))); }

__device__ __forceinline__ void gates_one(float ze, float za, float zb, float zm,
                                          const GateConsts& c, float& alpha, float& mu,
                                          float& eta, float& beta)
{
    eta = 2.f * rcp(1.f + ex2(ze * c.eta_scale));
    const float x = c.s * eta;
    const float x2 = x * x;
    const float amax = rcp(1.f + x2);      // cos^2(arctan x)
    const float bmax = x2 * amax;          // sin^2(arctan x)
    alpha = amax * ex2(-c.a * sp2(fmaf(za, LOG2E, c.bL)));
    beta = bmax * rcp(1.f + ex2(-zb * LOG2E));
    mu = ex2(fmaxf(-c.a * sp2(fmaf(zm, LOG2E, c.bL)), c.floorL));
}

template <int V>
__global__ __launch_bounds__(256) void gates_kernel(const float* __restrict__ z_eta,
                                                    const float* __restrict__ z_alpha,
                                                    const float* __restrict__ z_beta,
                                                    const float* __restrict__ z_mu, size_t n,
                                                    GateConsts c, float* __restrict__ alpha,
                                                    float* __restrict__ mu,
                                                    float* __restrict__ eta,
                                                    float* __restrict__ beta)
{
    using vec = fvec<V>;
    const size_t nv = n / V;   // whole vectors
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv; i += stride) {
        const vec ze = reinterpret_cast<const vec*>(z_eta)[i];
        const vec za = reinterpret_cast<const vec*>(z_alpha)[i];
        const vec zb = reinterpret_cast<const vec*>(z_beta)[i];
        const vec zm = reinterpret_cast<const vec*>(z_mu)[i];
        vec a, m, e, b;
#pragma unroll
        for (int j = 0; j < V; ++j) {
            float ga, gm, ge, gb;
            gates_one(ze[j], za[j], zb[j], zm[j], c, ga, gm, ge, gb);
            a[j] = ga;
            m[j] = gm;
            e[j] = ge;
            b[j] = gb;
        }
        reinterpret_cast<vec*>(alpha)[i] = a;
        reinterpret_cast<vec*>(mu)[i] = m;
        reinterpret_cast<vec*>(eta)[i] = e;
        reinterpret_cast<vec*>(beta)[i] = b;
    }
    // the last n % V elements, one per thread of the first workgroup
    if (V > 1 && blockIdx.x == 0 && threadIdx.x < n % V) {
        const size_t i = V * nv + threadIdx.x;
        gates_one(z_eta[i], z_alpha[i], z_beta[i], z_mu[i], c, alpha[i], mu[i], eta[i], beta[i]);
    }
}

constexpr unsigned GATES_MAX_BLOCKS = 16384;

template <int V>
hipError_t launch_gates_v(const float* z_eta, const float* z_alpha, const float* z_beta,
                          const float* z_mu, size_t n, const GateConsts& c, float* alpha,
                          float* mu, float* eta, float* beta, hipStream_t stream)
{
    const size_t nv = n / V;
    // enough workgroups to fill the GPU several times over, then grid-stride
    const size_t want = (nv + 255) / 256;
    const unsigned blocks =
        (unsigned)(want < 1 ? 1 : want > GATES_MAX_BLOCKS ? GATES_MAX_BLOCKS : want);
    hipLaunchKernelGGL(gates_kernel<V>, dim3(blocks), dim3(256), 0, stream, z_eta, z_alpha,
                       z_beta, z_mu, n, c, alpha, mu, eta, beta);
    return hipGetLastError();
}

GateConsts gate_consts(float tau, float s, float a, float b, float log_mu_min)
{
    return GateConsts{-2.f * LOG2E / tau, s, a, b * LOG2E, log_mu_min * LOG2E};
}

}  // namespace

// Host entry used by the C ABI layer; arguments are validated there.
hipError_t launch_gates(const float* z_eta, const float* z_alpha, const float* z_beta,
                        const float* z_mu, size_t n, float tau, float s, float a, float b,
                        float log_mu_min, float* alpha, float* mu, float* eta, float* beta,
                        hipStream_t stream)
{
    // two values per thread and array (8-byte accesses): at a layer's size
    // (B T H = 2^19) the fastest of 1, 2 and 4 per thread (3.5 us against
    // 4.7 and 3.4-4.6 us, back to back); at 2^23 within 3% of the best
    return launch_gates_v<2>(z_eta, z_alpha, z_beta, z_mu, n, gate_consts(tau, s, a, b, log_mu_min),
                             alpha, mu, eta, beta, stream);
}

}  // namespace mdn
