/*
 * libmdn.h -- C ABI of libmdn, a gfx950 (MI355X) implementation of the
 * Momentum DeltaNet (MDN) memory core: its chunkwise-parallel forward pass
 * and its recurrent decode step.
 *
 * The operation (per batch entry b and head h, tokens t = 1..T):
 *     vt_t = v_t - alpha_t S_{t-1}^T k_t
 *     M_t  = mu_t M_{t-1} - eta_t k_t vt_t^T
 *     S_t  = alpha_t S_{t-1} - beta_t M_t
 *     o_t  = S_t^T q_t
 * with S, M in R^{Dk x Dv}.  This is the two-state recurrence of "MDN:
 * Parallelizing Stepwise Momentum for Delta Linear Attention" (slides),
 * Sec. 3.1 Eqs. (3)-(5); the update-step gate beta is optional (a NULL beta
 * means beta = 1, the form the slides' chunk equations are written in, and
 * then runs exactly the arithmetic an all-ones beta runs).  The forward
 * pass evaluates it chunk by chunk as in the same slides' Eqs. (7)-(9),
 * (15)-(18) and (40)-(42) (Appendix C forms, residual mask shifted one row
 * as in the backup frame "a one-row shift is essential for causality"),
 * which is exact in real arithmetic; the decode step applies one token.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing and keeps no per-call state; it is reentrant.
 *  - Calls only enqueue work on `stream` and never synchronise; results are
 *    valid once the stream has been synchronised.
 *  - Arguments are validated on the host before any launch; on an error
 *    nothing is launched and the status says why.  MDN_ERR_HIP reports a
 *    failed launch.  Device data is never inspected: gate values are not
 *    range-checked and non-finite values propagate.
 *  - Pointers must be 16-byte aligned (MDN_ERR_ALIGN otherwise).
 *  - No query scaling is applied: fold any d_k^{-1/2} into q.
 *  - Supported head sizes: Dk, Dv in {64, 128}; chunk length 64.
 *
 * Layouts (row-major, C order):
 *    q, k    [B, T, H, Dk]     dtype `dt`
 *    v, O    [B, T, H, Dv]     dtype `dt`
 *    alpha, mu, eta, beta  [B, T, H] float32 (beta may be NULL)
 *    S0, M0, S_T, M_T [B, H, Dk, Dv] float32
 *  Decode: q, k [N, H, Dk]; v, o [N, H, Dv]; gates [N, H]; S, M [N, H, Dk, Dv].
 */
#ifndef LIBMDN_H
#define LIBMDN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MDN_OK = 0,
    MDN_ERR_NULL = 1,        /* a required pointer is NULL                       */
    MDN_ERR_SHAPE = 2,       /* a size is negative or a product overflows        */
    MDN_ERR_UNSUPPORTED = 3, /* head size, chunk length or dtype not supported    */
    MDN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                  */
    MDN_ERR_ALIAS = 5,       /* an output overlaps an input (other than in place) */
    MDN_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required           */
    MDN_ERR_HIP = 7          /* a HIP launch failed                               */
} mdn_status;

typedef enum {
    MDN_F32 = 0,  /* q, k, v and the output in float32  */
    MDN_BF16 = 1  /* q, k, v and the output in bfloat16 */
} mdn_dtype;

/*
 * How the bf16 forward partitions the carried state over workgroups.  The
 * scan over chunks is sequential, so its parallelism is the number of state
 * tiles in flight (times the number of segments, for the segment scan):
 *   MDN_FWD_COLUMN_TILES  one workgroup per 64 value columns of a head, each
 *                         wavefront owning 16 columns and all Dk rows.
 *                         mdn_chunk_fwd runs one fused kernel that also forms
 *                         T and A on chip; mdn_chunk_fwd_scan runs the
 *                         column-tiled scan.
 *   MDN_FWD_ROW_SPLIT     one workgroup per 16 value columns (4x the
 *                         workgroups), its Dk/32 wavefronts splitting the
 *                         rows and exchanging partial products in LDS.
 *                         mdn_chunk_fwd runs the two phases below
 *                         (mdn_chunk_fwd_prepare's kernel, then this scan).
 *                         It does not produce the residuals: a call with
 *                         Vt != NULL runs the column-tiled kernels.
 *   MDN_FWD_SEGMENTS      the sequence cut into nseg >= 3 segments of at
 *                         least 8 chunks.  A segment's exit state is affine
 *                         in its entry state (the chunk recurrence of
 *                         "MDN: Parallelizing Stepwise Momentum for Delta
 *                         Linear Attention", frame "Chunk outputs combine
 *                         incoming states and local writes"): its exit from
 *                         a zero entry plus a linear map of the entry, found
 *                         by running the recurrence with V = 0 from the
 *                         identity's columns.  Pass 1 runs segment 0 from
 *                         the entry state beside the maps of segments
 *                         1 .. nseg - 2; a small kernel chains them into the
 *                         entry state of every segment; pass 2 runs segments
 *                         1 .. nseg - 1 from those, so each pass walks
 *                         1 / nseg of the chunks.  nseg is the largest with
 *                         both passes within one workgroup per compute unit;
 *                         where none of 3 or more fits (many heads, or fewer
 *                         than 24 chunks) the column tiles run.  It does not
 *                         produce the residuals (Vt != NULL: column tiles).
 *   MDN_FWD_AUTO          (the default) the segment scan where three or more
 *                         segments of at least 16 chunks fit, at least 8
 *                         with mu NULL (few heads and long sequences;
 *                         measured on MI355X at d = 128 it took 0.23 to 0.90
 *                         of the other paths' time there; with mu and 8 to
 *                         11 chunks per segment about as long as theirs,
 *                         without mu 0.84 to 0.90); otherwise the row split when the layer
 *                         has at most 32 column tiles, B * H * (Dv / 64) <=
 *                         32, where it measured faster than the column tiles
 *                         (at 64 tiles the two are about even, at 128 the
 *                         column tiles take half the time); otherwise the
 *                         column tiles.
 * All paths evaluate the same equations; their results agree to rounding,
 * not bit for bit.  MDN_F32 always runs the two-phase path.
 */
typedef enum {
    MDN_FWD_AUTO = 0,
    MDN_FWD_COLUMN_TILES = 1,
    MDN_FWD_ROW_SPLIT = 2,
    MDN_FWD_SEGMENTS = 3
} mdn_fwd_path;

/*
 * Sets the process-wide forward path for every later call (on any device
 * and thread) and returns the previous setting; an unknown value changes
 * nothing and returns -1.  Meant for benchmarking and testing both
 * partitions: a workspace sized by mdn_chunk_fwd_workspace_bytes under one
 * setting may be too small under another (MDN_ERR_WORKSPACE, nothing
 * launched).
 */
int mdn_set_fwd_path(int path);

/*
 * The number of segments a bf16 mdn_chunk_fwd call of this shape (with_mu:
 * mu is given; no residuals asked for) runs the segment scan with under the
 * current mdn_set_fwd_path setting; 0 when it runs another path.  Host only:
 * no device is touched.  Negative or unsupported sizes return 0.
 */
int mdn_fwd_segment_count(int B, int T, int H, int Dk, int Dv, int with_mu);

/*
 * Bytes of device workspace mdn_chunk_fwd needs for this problem under the
 * current mdn_set_fwd_path setting.  When dt = MDN_BF16 selects the
 * column tiles, the forward keeps the chunk-local matrices T and A on chip
 * and needs only per-chunk coefficient tables (6656 bytes per chunk of 64
 * tokens and head: the gates, the block products and boundary values of
 * the slides' Gamma of Eqs. (7)-(9), the lower triangles of its 16 x 16
 * diagonal blocks and the six coefficient rows the scan reads).  With
 * MDN_F32, and with the row split, it runs as the two phases below and
 * needs what mdn_chunk_fwd_split_workspace_bytes returns (the larger; it
 * is returned whenever the row split may run, so it also covers a call
 * that asks for Vt).  Returns 0 for unsupported or invalid sizes and when
 * no work is needed (B, T or H is 0).
 */
size_t mdn_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                     mdn_dtype dt);

/*
 * Bytes of device workspace the split entry points mdn_chunk_fwd_prepare /
 * mdn_chunk_fwd_scan exchange: per chunk the coefficient vectors and the
 * chunk-local matrices T = L^{-1} and A of the slides' Eqs. (15)-(18) and
 * (40)-(42).  0 for unsupported or invalid sizes and when B, T or H is 0.
 */
size_t mdn_chunk_fwd_split_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                           mdn_dtype dt);

/*
 * Chunkwise MDN forward over T tokens.
 *   q, k, v          inputs, layouts above, dtype dt.
 *   alpha, mu, eta   per-token, per-head gates (float32).  Any finite values
 *                    are accepted; mu = 0 is the gated delta rule and
 *                    additionally alpha = 1 is DeltaNet.  mu may be NULL,
 *                    meaning mu = 0: the momentum then never feeds the memory
 *                    and a kernel without the momentum products runs (M0 is
 *                    not read; M_T receives the last token's own write
 *                    -eta_T k_T vt_T^T).
 *   beta             the update-step gate (float32, same layout), or NULL for
 *                    beta = 1.
 *   S0, M0           initial memory and momentum (float32); NULL = zero.
 *   O                output o_t for every token (dtype dt); must not overlap
 *                    any input.
 *   Vt               NULL, or [B, T, H, Dv] (dtype dt): receives every token's
 *                    residual vt_t = v_t - alpha_t S_{t-1}^T k_t (the chunk
 *                    form's Vt = L^{-1} R), the activations the slides' frame
 *                    "The implementation trades saved residuals for
 *                    throughput" keeps for the backward pass (mdn_chunk_bwd
 *                    then rebuilds the states from them without the solve).
 *                    Overlaps nothing.
 *   S_T, M_T         final memory and momentum (float32); NULL = not written.
 *                    S_T may be exactly S0 and M_T exactly M0 (in place); any
 *                    other overlap is MDN_ERR_ALIAS.
 *   chunk            must be 64.  T need not be a multiple of it: the last
 *                    chunk is then partial.
 *   workspace        device buffer of at least
 *                    mdn_chunk_fwd_workspace_bytes(...) bytes, owned by the
 *                    caller; its contents on entry do not matter.
 * B, H >= 0 and T >= 0.  With T = 0, S_T/M_T receive S0/M0 (zeros if NULL)
 * and O is untouched; with B = 0 or H = 0 nothing is launched.
 */
mdn_status mdn_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                         const float* mu, const float* eta, const float* beta, const float* S0,
                         const float* M0, void* O, void* Vt, float* S_T, float* M_T, int B,
                         int T, int H, int Dk, int Dv, int chunk, mdn_dtype dt, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * mdn_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, rules and results as
 * mdn_chunk_fwd (the same kernels run, so the outputs are bitwise those of
 * mdn_chunk_fwd, except in the row-split case below); the workspace is
 * instead a file-scope device array of
 * MDN_NOALLOC_SCRATCH_BYTES (64 MiB) in the library, one per GPU, loaded with
 * the library's code on that GPU and held until the process ends.  Its
 * address is looked up once per GPU on the first call there.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * Limits and errors:
 *   - when mdn_set_fwd_path selects the row split (see mdn_fwd_path) but its
 *     workspace (18,432 bytes per chunk of 64 tokens and head) exceeds the
 *     array, the column tiles run instead;
 *   - a problem whose workspace for the path it runs exceeds
 *     MDN_NOALLOC_SCRATCH_BYTES returns MDN_ERR_WORKSPACE before anything is
 *     enqueued (bf16 column tiles: 6,656 bytes per chunk of 64 tokens and
 *     head, so up to 10,082 chunks, e.g. B8 H16 T4096; fp32: the two-phase
 *     workspace);
 *   - MDN_ERR_HIP if the array's address cannot be looked up.
 * Every call on one GPU shares that GPU's array, and a call leaves its
 * contents behind: calls that overlap in time on one GPU (on different
 * streams, or from different threads without ordering) race and give wrong
 * results.  Calls ordered on one stream are safe.  No kernel relies on the
 * array's contents on entry.
 */
#define MDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

mdn_status mdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const float* alpha, const float* mu, const float* eta,
                                 const float* beta, const float* S0, const float* M0, void* O,
                                 void* Vt, float* S_T, float* M_T, int B, int T, int H, int Dk,
                                 int Dv, int chunk, mdn_dtype dt, hipStream_t stream);

/*
 * The forward as two separate phases, for callers that want to run the
 * chunk-local phase ahead of the scan (for instance on another stream) or
 * time them apart.  The reading notes on the MDN paper (Sec. 2.4) point out
 * that T = [I + (P Khat^T) o Gamma^-]^{-1} and the scalar coefficients depend
 * only on chunk-local inputs, while the carried state enters afterwards; the
 * split follows that.  mdn_chunk_fwd_prepare(...) followed by
 * mdn_chunk_fwd_scan(...) on one stream with one workspace computes what
 * mdn_chunk_fwd(...) computes (for MDN_F32 it is exactly how mdn_chunk_fwd
 * runs; for MDN_BF16 mdn_chunk_fwd runs a coefficient kernel and one fused
 * kernel that evaluate the same equations, so the two agree to rounding,
 * not bit for bit).
 *
 * mdn_chunk_fwd_prepare: per chunk, the coefficients (abar, mubar, b, Gamma;
 *   slides Eqs. (7)-(9)), T = L^{-1} (Eqs. (15)-(18)) and
 *   A = (Q Khat^T) o Gamma (Eqs. (40)-(42)), written to `workspace`.
 *   Reads q, k and the gates only (layouts and the optional beta as for
 *   mdn_chunk_fwd; Dk is the
 *   head size of q and k).  The workspace must hold at least
 *   mdn_chunk_fwd_split_workspace_bytes(B, T, H, Dk, Dv, chunk, dt) bytes
 *   (the size does not depend on Dk or Dv) and must not overlap any input.
 *   T = 0, B = 0 or H = 0: nothing is launched.
 *
 * mdn_chunk_fwd_scan: the sequential part (residuals, outputs and the
 *   carried state pair), reading q, k, v, S0/M0 and the workspace a previous
 *   mdn_chunk_fwd_prepare with the same B, T, H, Dk, chunk and dt filled on
 *   the same stream (or after it, in stream order).  Output rules as for
 *   mdn_chunk_fwd.
 * Both return the same status codes as mdn_chunk_fwd for the same errors.
 */
mdn_status mdn_chunk_fwd_prepare(const void* q, const void* k, const float* alpha,
                                 const float* mu, const float* eta, const float* beta, int B,
                                 int T, int H, int Dk, int chunk, mdn_dtype dt, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

mdn_status mdn_chunk_fwd_scan(const void* q, const void* k, const void* v, const float* S0,
                              const float* M0, void* O, float* S_T, float* M_T, int B, int T,
                              int H, int Dk, int Dv, int chunk, mdn_dtype dt,
                              const void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One recurrent decode step for N independent sequences (the recurrence
 * above with T = 1; the slides' Sec. 3.1 notes that decoding keeps the
 * fixed-size pair S, M).
 *   q, k [N, H, Dk], v [N, H, Dv]    this step's token (dtype dt).
 *   alpha, mu, eta [N, H]            this step's gates (float32).  mu may be
 *                                    NULL, meaning mu = 0: M is then not
 *                                    read and may be NULL; if it is not, it
 *                                    receives the step's -eta k vt^T.
 *   beta [N, H] or NULL              this step's update-step gate (NULL: 1).
 *   S, M [N, H, Dk, Dv]              state, read and updated IN PLACE (float32).
 *   o [N, H, Dv]                     output (dtype dt); must not overlap any
 *                                    other argument.
 * N, H >= 0; N = 0 or H = 0 launches nothing.
 */
mdn_status mdn_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                           const float* mu, const float* eta, const float* beta, float* S,
                           float* M, void* o, int N, int H, int Dk, int Dv, mdn_dtype dt,
                           hipStream_t stream);

/*
 * Backward pass of mdn_chunk_fwd: the gradients of a loss L through the
 * forward, given dO = dL/dO and dS_T, dM_T = dL/dS_T, dL/dM_T.  The pages
 * ("MDN: Parallelizing Stepwise Momentum for Delta Linear Attention"
 * (slides), frame "The implementation trades saved residuals for
 * throughput"; the paper's Sec. 3.1 and Appendix E) describe the strategy --
 * rebuild the states for the gradients instead of storing every state pair --
 * but print no gradient formulas; these are the chain rule through the chunk
 * equations of mdn_chunk_fwd, chunk by chunk from the last.  The call takes
 * the residuals Vt the forward saved (or recomputes them when Vt is NULL) and
 * keeps each chunk's entry state and exit-state gradients in the workspace
 * while it runs.  All sums are fp32.  For dt = MDN_F32 every product is
 * fp32; for dt = MDN_BF16 the stored states are bf16 and most products run on
 * bf16 matrix instructions, with operands that are bf16 inputs, rounded to
 * bf16, or split into a bf16 head and remainder (each kernel's comments say
 * which), so each gradient tensor is accurate to about 1e-2 of its largest
 * magnitude.
 *   q, k, v, alpha, mu, eta, beta, S0, M0, B, T, H, Dk, Dv, chunk, dt:
 *                         exactly as given to mdn_chunk_fwd (mu, beta, S0, M0
 *                         may be NULL with the same meaning).
 *   dO [B, T, H, Dv]       dtype dt.
 *   dS_T, dM_T [B, H, Dk, Dv] or NULL (zero), float32.
 *   Vt [B, T, H, Dv] (dtype dt) or NULL: the residuals mdn_chunk_fwd saved
 *                          for these inputs.  Given, the states are rebuilt
 *                          from them (no solve); NULL recomputes them.
 * Outputs, all float32, each overwritten:
 *   dq, dk [B, T, H, Dk]; dv [B, T, H, Dv];
 *   dalpha, deta [B, T, H]; dmu [B, T, H] (only when mu is given; may be
 *   NULL otherwise); dbeta [B, T, H] (only when beta is given; may be NULL
 *   otherwise); dS0, dM0 [B, H, Dk, Dv] or NULL (not returned).
 * Every pointer is a device pointer aligned to 16 bytes; no output may
 * overlap an input, another output or the workspace.  Workspace:
 * mdn_chunk_bwd_workspace_bytes: T and A of every chunk (dtype dt), the
 * coefficient rows (float32), each chunk's entry-state pair and exit-state
 * gradient pair (dtype dt: bf16 for MDN_BF16, float32 for MDN_F32) and each
 * chunk's recomputed residuals (float32, written only when Vt is NULL); its
 * contents on entry do not matter.  T = 0 copies dS_T, dM_T to dS0, dM0.
 * Enqueued on `stream`.
 */
size_t mdn_chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                     mdn_dtype dt);

mdn_status mdn_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                         const float* mu, const float* eta, const float* beta, const float* S0,
                         const float* M0, const void* dO, const float* dS_T, const float* dM_T,
                         const void* Vt, float* dq, float* dk, float* dv, float* dalpha,
                         float* dmu, float* deta,
                         float* dbeta, float* dS0, float* dM0, int B, int T, int H, int Dk,
                         int Dv, int chunk, mdn_dtype dt, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * The elementwise steps around the core, each one pass over HBM ("MDN:
 * Parallelizing Stepwise Momentum for Delta Linear Attention" (slides), frame
 * "The memory sits inside a familiar language-model block"; the paper's
 * Sec. 3.3 and Fig. 3).
 *
 * mdn_qk_prologue: the Comba query correction and the L2 normalisation of
 * queries and keys, per token and head over Dk:
 *     q' = q - d_h k,   q_out = q' / sqrt(|q'|^2 + eps),   k_out = k / sqrt(|k|^2 + eps)
 *   q, k, q_out, k_out [rows, H, Dk] (dtype dt; rows = tokens, e.g. B T);
 *   d [H] float32 or NULL (no correction).
 * mdn_output_epilogue: the gated output norm before the output projection,
 * per token and head over Dv:
 *     y = sigmoid(g) * (o / sqrt(mean(o^2) + eps)) * w
 *   o, g, y [rows, H, Dv] (dtype dt; g is the caller's gate projection);
 *   w [Dv] float32 shared by the heads, or NULL (ones).
 * Dk, Dv in {64, 128}; eps finite and > 0 (MDN_ERR_UNSUPPORTED otherwise).
 * Device pointers aligned to 16 bytes.  An output may be its own input
 * exactly (q_out = q, k_out = k, y = o: in place) and must overlap nothing
 * else (MDN_ERR_ALIAS).  rows = 0 or H = 0 launches nothing.  Enqueued on
 * `stream`; the caller owns every buffer.
 */
mdn_status mdn_qk_prologue(const void* q, const void* k, const float* d, void* q_out,
                           void* k_out, size_t rows, int H, int Dk, float eps, mdn_dtype dt,
                           hipStream_t stream);

mdn_status mdn_output_epilogue(const void* o, const void* g, const float* w, void* y,
                               size_t rows, int H, int Dv, float eps, mdn_dtype dt,
                               hipStream_t stream);

/*
 * MDN's coupled gate parameterisation ("MDN: Parallelizing Stepwise Momentum
 * for Delta Linear Attention" (slides), frame "Coupled gates restrict the
 * spectral region", the paper's Sec. 3.3), from logits the caller computes
 * (its projections W x_t of the layer input) to the gates of the recurrence:
 *     eta   = 1 + tanh(z_eta / tau)
 *     theta = arctan(s eta),  alpha_max = cos^2 theta,  beta_max = sin^2 theta
 *     log alpha = f(z_alpha) + log alpha_max
 *     beta      = sigmoid(z_beta) beta_max
 *     log mu    = max(f(z_mu), log_mu_min),      f(z) = -a softplus(z + b)
 * so that eta is in (0, 2) and, for a >= 0, alpha + beta <= 1.  The slides
 * give tau = sqrt(d_in / h) as the paper's default and log_mu_min = -2 for
 * the reported experiments; a, b and s are the caller's.
 *   z_eta, z_alpha, z_beta, z_mu    n logits each (float32, any layout, one
 *                                   value per token and head).
 *   alpha, mu, eta, beta            n gates each (float32, same order), in
 *                                   the form mdn_chunk_fwd and
 *                                   mdn_decode_step take them.
 * All eight are device pointers aligned to 16 bytes (MDN_ERR_ALIGN), none
 * NULL (MDN_ERR_NULL) unless n = 0, which launches nothing.  No output may
 * overlap another output or an input (MDN_ERR_ALIAS); inputs may share
 * memory.  tau must be positive and every parameter finite
 * (MDN_ERR_UNSUPPORTED otherwise).  Enqueued on `stream`; the caller owns
 * every buffer.
 */
typedef struct {
    float tau;          /* temperature of eta                              */
    float s;            /* angle scale of theta                            */
    float a, b;         /* f(z) = -a softplus(z + b), for alpha and mu     */
    float log_mu_min;   /* floor of log mu                                 */
} mdn_gate_params;

mdn_status mdn_gates_from_logits(const float* z_eta, const float* z_alpha, const float* z_beta,
                                 const float* z_mu, size_t n, mdn_gate_params params,
                                 float* alpha, float* mu, float* eta, float* beta,
                                 hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* mdn_status_string(mdn_status s);

#ifdef __cplusplus
}
#endif

#endif /* LIBMDN_H */
