// api.hip -- the libmdn C ABI: host-side validation and dispatch.
//
// Every check happens here, before anything is launched; an error status
// means nothing was enqueued.  Device data is never inspected.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <initializer_list>
#include <mutex>

#include "../../include/libmdn.h"

namespace mdn {
size_t chunk_workspace_bytes(int B, int T, int H, bool bf16);
hipError_t launch_chunk_prepare(const void* q, const void* k, const float* alpha, const float* mu,
                                const float* eta, const float* beta, int B, int T, int H, int Dk,
                                bool bf16, void* workspace, hipStream_t stream);
size_t chunk_fused_workspace_bytes(size_t nchunks);
int chunk_seg_count(int B, int T, int H, int Dk, int Dv, bool mom, int min_ncs);
size_t chunk_seg_workspace_bytes(int B, int T, int H, int Dk, int Dv, int nseg, bool mom);
hipError_t launch_chunk_fused_seg(const void* q, const void* k, const void* v,
                                  const float* alpha, const float* mu, const float* eta,
                                  const float* beta, const float* S0, const float* M0, void* O,
                                  float* ST, float* MT, int B, int T, int H, int Dk, int Dv,
                                  int nseg, void* workspace, hipStream_t stream);
hipError_t launch_chunk_fused(const void* q, const void* k, const void* v, const float* alpha,
                              const float* mu, const float* eta, const float* beta,
                              const float* S0, const float* M0, void* O, void* Vto, float* ST,
                              float* MT, int B, int T, int H, int Dk, int Dv, void* workspace,
                              hipStream_t stream);
hipError_t launch_chunk_scan(const void* q, const void* k, const void* v, const float* S0,
                             const float* M0, void* O, void* Vto, float* ST, float* MT, int B,
                             int T, int H, int Dk, int Dv, bool bf16, bool row_split,
                             bool momentum, const void* workspace, hipStream_t stream);
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* alpha,
                         const float* mu, const float* eta, const float* beta, float* S, float* M,
                         void* o, int heads, int Dk, int Dv, bool bf16, hipStream_t stream);
size_t chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, bool bf16);
hipError_t launch_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                            const float* mu, const float* eta, const float* beta, const float* S0,
                            const float* M0, const void* dO, const float* dST, const float* dMT,
                            const void* Vsaved, float* dq, float* dk, float* dv, float* dalpha,
                            float* dmu, float* deta, float* dbeta, float* dS0, float* dM0, int B,
                            int T, int H, int Dk, int Dv, bool bf16, void* workspace,
                            hipStream_t stream);
hipError_t launch_state_copy(const float* src, float* dst, size_t count, hipStream_t stream);
hipError_t launch_qk_prologue(const void* q, const void* k, const float* dcorr, void* qo,
                              void* ko, size_t rows, int H, int D, bool bf16, float eps,
                              hipStream_t stream);
hipError_t launch_output_epilogue(const void* o, const void* g, const float* w, void* y,
                                  size_t rows, int D, bool bf16, float eps, hipStream_t stream);
hipError_t launch_gates(const float* z_eta, const float* z_alpha, const float* z_beta,
                        const float* z_mu, size_t n, float tau, float s, float a, float b,
                        float log_mu_min, float* alpha, float* mu, float* eta, float* beta,
                        hipStream_t stream);
}  // namespace mdn

namespace {

struct Span {
    uintptr_t lo = 0, hi = 0;   // [lo, hi); empty when lo == hi
};

Span span(const void* p, size_t bytes)
{
    Span s;
    if (p && bytes) {
        s.lo = reinterpret_cast<uintptr_t>(p);
        s.hi = s.lo + bytes;
    }
    return s;
}

bool overlap(const Span& a, const Span& b)
{
    return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }

// a * b * c * d without overflow past 2^62 (plenty for any device buffer)
bool mul_ok(size_t a, size_t b, size_t c, size_t d, size_t* out)
{
    const size_t lim = (size_t)1 << 62;
    size_t x = a;
    for (size_t f : {b, c, d}) {
        if (f != 0 && x > lim / f) return false;
        x *= f;
    }
    *out = x;
    return true;
}

// The bf16 forward's partition of the state (mdn_set_fwd_path).
std::atomic<int> fwd_path{MDN_FWD_AUTO};

// Under MDN_FWD_AUTO the row split runs up to this many 64-column head tiles
// (an eighth of the 256 compute units).  Measured on MI355X (d = 128): at 8
// to 32 tiles and 4K to 16K tokens the row split took 0.84-0.96 of the column
// tiles' time, at 64 tiles 0.95-1.09 and at 128 tiles about 2x.
constexpr size_t ROW_SPLIT_MAX_TILES = 32;

// True when a bf16 forward of this shape runs the row-split scan; `want_vt`:
// the caller asked for the residuals, which only the column tiles store.
bool row_split_for(int B, int H, int Dv, mdn_dtype dt, bool want_vt)
{
    if (dt != MDN_BF16 || want_vt || B <= 0 || H <= 0) return false;
    const int p = fwd_path.load(std::memory_order_relaxed);
    if (p == MDN_FWD_COLUMN_TILES || p == MDN_FWD_SEGMENTS) return false;
    if (p == MDN_FWD_ROW_SPLIT) return true;
    return (size_t)B * (size_t)H * (size_t)(Dv / 64) <= ROW_SPLIT_MAX_TILES;
}

// Under MDN_FWD_AUTO the segment scan runs where it has three or more
// segments of at least this many chunks.  Measured on MI355X (d = 128): with
// 16 to 64 chunks per segment it took 0.11 to 0.9 of the best other path's
// time (at B1 H16: T4096 0.90, T16384 0.67, with mu = 0 0.69 and 0.59; at
// B1 H2 T65536 0.23).  With 8 to 11 chunks per segment (B1 H16 T2048, B4 H8
// T2048) it took 0.97 and 1.02 of the best other path's time with mu, and
// 0.84 and 0.90 without (a transition without momentum has a third fewer
// columns), so without mu the bar is lower.
constexpr int SEG_AUTO_MIN_CHUNKS = 16;
constexpr int SEG_AUTO_MIN_CHUNKS_NO_MU = 8;
constexpr int SEG_MIN_CHUNKS = 8;   // MDN_FWD_SEGMENTS

// The number of segments when a bf16 forward of this shape runs the segment
// scan, else 0; `mom`: mu is given.
int segments_for(int B, int T, int H, int Dk, int Dv, mdn_dtype dt, bool want_vt, bool mom)
{
    if (dt != MDN_BF16 || want_vt || B <= 0 || H <= 0 || T <= 0) return 0;
    if (!head_dim_ok(Dk) || !head_dim_ok(Dv)) return 0;
    const int p = fwd_path.load(std::memory_order_relaxed);
    if (p != MDN_FWD_SEGMENTS && p != MDN_FWD_AUTO) return 0;
    const int auto_min = mom ? SEG_AUTO_MIN_CHUNKS : SEG_AUTO_MIN_CHUNKS_NO_MU;
    const int n = mdn::chunk_seg_count(B, T, H, Dk, Dv, mom,
                                       p == MDN_FWD_AUTO ? auto_min : SEG_MIN_CHUNKS);
    return n >= 3 ? n : 0;
}

}  // namespace

extern "C" {

const char* mdn_status_string(mdn_status s)
{
    switch (s) {
    case MDN_OK: return "MDN_OK";
    case MDN_ERR_NULL: return "MDN_ERR_NULL: a required pointer is NULL";
    case MDN_ERR_SHAPE: return "MDN_ERR_SHAPE: a size is negative or too large";
    case MDN_ERR_UNSUPPORTED: return "MDN_ERR_UNSUPPORTED: head size, chunk or dtype not supported";
    case MDN_ERR_ALIGN: return "MDN_ERR_ALIGN: a pointer is not 16-byte aligned";
    case MDN_ERR_ALIAS: return "MDN_ERR_ALIAS: an output overlaps another argument";
    case MDN_ERR_WORKSPACE: return "MDN_ERR_WORKSPACE: workspace missing or too small";
    case MDN_ERR_HIP: return "MDN_ERR_HIP: a HIP launch failed";
    }
    return "unknown mdn_status";
}

static size_t split_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk, mdn_dtype dt)
{
    if (B <= 0 || T <= 0 || H <= 0) return 0;
    if (!head_dim_ok(Dk) || !head_dim_ok(Dv) || chunk != 64) return 0;
    if (dt != MDN_F32 && dt != MDN_BF16) return 0;
    size_t tmp;
    if (!mul_ok((size_t)B, (size_t)T, (size_t)H, 1, &tmp)) return 0;
    return mdn::chunk_workspace_bytes(B, T, H, dt == MDN_BF16);
}

size_t mdn_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                     mdn_dtype dt)
{
    // the bf16 column tiles keep T and A on chip and need only the per-chunk
    // coefficient tables
    const size_t split = split_workspace_bytes(B, T, H, Dk, Dv, chunk, dt);
    if (split == 0 || dt != MDN_BF16) return split;
    // the column tiles (a call that asks for the residuals runs them), the
    // segment scan where it runs with or without mu, the row split where a
    // call without segments runs it
    size_t need = mdn::chunk_fused_workspace_bytes((size_t)B * H * (((size_t)T + 63) / 64));
    bool every_call_segments = true;
    for (bool mom : {false, true}) {
        const int n = segments_for(B, T, H, Dk, Dv, dt, false, mom);
        if (n > 0)
            need = std::max(need, mdn::chunk_seg_workspace_bytes(B, T, H, Dk, Dv, n, mom));
        else
            every_call_segments = false;
    }
    if (!every_call_segments && row_split_for(B, H, Dv, dt, false)) need = std::max(need, split);
    return need;
}

int mdn_fwd_segment_count(int B, int T, int H, int Dk, int Dv, int with_mu)
{
    return segments_for(B, T, H, Dk, Dv, MDN_BF16, false, with_mu != 0);
}

int mdn_set_fwd_path(int path)
{
    if (path != MDN_FWD_AUTO && path != MDN_FWD_COLUMN_TILES && path != MDN_FWD_ROW_SPLIT &&
        path != MDN_FWD_SEGMENTS)
        return -1;
    return fwd_path.exchange(path);
}

size_t mdn_chunk_fwd_split_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                           mdn_dtype dt)
{
    return split_workspace_bytes(B, T, H, Dk, Dv, chunk, dt);
}

}  // extern "C"

namespace {

enum Phase { PREPARE = 1, SCAN = 2, BOTH = 3 };

struct FwdArgs {
    const void *q, *k, *v;
    const float *alpha, *mu, *eta, *beta, *S0, *M0;   // beta may be NULL
    void* O;
    void* Vt;   // optional: the residuals of every token (mdn_chunk_fwd only)
    float *S_T, *M_T;
    int B, T, H, Dk, Dv, chunk;
    mdn_dtype dt;
    const void* ws;
    size_t ws_bytes;
    // the workspace is the library's own per-device scratch array, resolved
    // after validation: ws_bytes is its capacity, and it overlaps no
    // caller buffer
    bool static_ws = false;
    // bf16: the row-split scan runs (after the prepare kernel when phase is
    // BOTH) instead of the column-tiled kernels
    bool row_split = false;
    // bf16, phase BOTH: the segment scan of this many segments (0: not)
    int nseg = 0;
};

// Every host-side check of the forward entry points.  `phase` says which
// arguments the call uses: the prepare phase reads q, k and the gates and
// writes the workspace; the scan reads q, k, v, the states and the workspace
// and writes O and the final states.
mdn_status validate_fwd(const FwdArgs& a, int phase, bool* no_work)
{
    *no_work = false;
    if (a.B < 0 || a.T < 0 || a.H < 0) return MDN_ERR_SHAPE;
    if (!head_dim_ok(a.Dk) || !head_dim_ok(a.Dv) || a.chunk != 64) return MDN_ERR_UNSUPPORTED;
    if (a.dt != MDN_F32 && a.dt != MDN_BF16) return MDN_ERR_UNSUPPORTED;
    if (a.B == 0 || a.H == 0 || (a.T == 0 && !(phase & SCAN))) {
        *no_work = true;
        return MDN_OK;
    }
    const size_t esz = a.dt == MDN_BF16 ? 2 : 4;
    size_t nqk, nv, ngate, nstate;
    if (!mul_ok((size_t)a.B, (size_t)a.T, (size_t)a.H, (size_t)a.Dk, &nqk) ||
        !mul_ok((size_t)a.B, (size_t)a.T, (size_t)a.H, (size_t)a.Dv, &nv) ||
        !mul_ok((size_t)a.B, (size_t)a.T, (size_t)a.H, 1, &ngate) ||
        !mul_ok((size_t)a.B, (size_t)a.H, (size_t)a.Dk, (size_t)a.Dv, &nstate))
        return MDN_ERR_SHAPE;
    // one workgroup per chunk (prepare) or per head tile (scan), 1-D grids
    if ((size_t)a.B * a.H * (((size_t)a.T + 63) / 64) > 0xffffffffu) return MDN_ERR_SHAPE;
    const bool tok = a.T > 0;
    if (tok && (!a.q || !a.k)) return MDN_ERR_NULL;
    // mu may be NULL: mu = 0 (the gated delta rule)
    if (tok && (phase & PREPARE) && (!a.alpha || !a.eta)) return MDN_ERR_NULL;
    if (tok && (phase & SCAN) && (!a.v || !a.O)) return MDN_ERR_NULL;

    const void* ptrs[] = {a.q, a.k, a.v, a.alpha, a.mu, a.eta, a.beta, a.S0, a.M0, a.O, a.Vt,
                          a.S_T, a.M_T, a.ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MDN_ERR_ALIGN;

    // the bf16 forward runs fused and needs only the per-chunk coefficient tables
    const bool fused = phase == BOTH && a.dt == MDN_BF16 && !a.row_split;
    const bool seg = fused && a.nseg >= 3;
    const size_t nchunks = (size_t)a.B * a.H * (((size_t)a.T + 63) / 64);
    const size_t need =
        !tok  ? 0
        : seg ? mdn::chunk_seg_workspace_bytes(a.B, a.T, a.H, a.Dk, a.Dv, a.nseg, a.mu != nullptr)
        : fused ? mdn::chunk_fused_workspace_bytes(nchunks)
                : mdn::chunk_workspace_bytes(a.B, a.T, a.H, a.dt == MDN_BF16);
    if (need > 0 && (a.static_ws ? need > a.ws_bytes : (!a.ws || a.ws_bytes < need)))
        return MDN_ERR_WORKSPACE;

    const size_t nt = tok ? 1 : 0;   // token arrays are empty when T == 0
    const bool prep = phase & PREPARE, scan = phase & SCAN;
    const Span sq = span(a.q, nt * nqk * esz), sk = span(a.k, nt * nqk * esz),
               sv = span(scan ? a.v : nullptr, nt * nv * esz),
               sa = span(prep ? a.alpha : nullptr, nt * ngate * 4),
               sm = span(prep ? a.mu : nullptr, nt * ngate * 4),
               se = span(prep ? a.eta : nullptr, nt * ngate * 4),
               sb = span(prep ? a.beta : nullptr, nt * ngate * 4),
               sS0 = span(scan ? a.S0 : nullptr, nstate * 4),
               sM0 = span(scan ? a.M0 : nullptr, nstate * 4),
               sO = span(scan ? a.O : nullptr, nt * nv * esz),
               sVt = span(scan ? a.Vt : nullptr, nt * nv * esz),
               sST = span(scan ? a.S_T : nullptr, nstate * 4),
               sMT = span(scan ? a.M_T : nullptr, nstate * 4),
               sW = span(a.static_ws ? nullptr : a.ws, need);
    const Span inputs[] = {sq, sk, sv, sa, sm, se, sb, sS0, sM0};
    // O and the workspace overlap nothing
    for (const Span& x : inputs)
        if (overlap(sO, x) || overlap(sW, x) || overlap(sVt, x)) return MDN_ERR_ALIAS;
    if (overlap(sO, sW) || overlap(sO, sST) || overlap(sO, sMT) || overlap(sW, sST) ||
        overlap(sW, sMT) || overlap(sST, sMT))
        return MDN_ERR_ALIAS;
    if (overlap(sVt, sO) || overlap(sVt, sW) || overlap(sVt, sST) || overlap(sVt, sMT))
        return MDN_ERR_ALIAS;
    // final states overlap no input, except exactly in place over their own
    // initial state
    for (int i = 0; i < 9; ++i) {
        if (overlap(sST, inputs[i]) && !(i == 7 && a.S_T == a.S0)) return MDN_ERR_ALIAS;
        if (overlap(sMT, inputs[i]) && !(i == 8 && a.M_T == a.M0)) return MDN_ERR_ALIAS;
    }
    return MDN_OK;
}

// Launches the forward's kernels for arguments validate_fwd accepted.
mdn_status launch_fwd(const FwdArgs& a, int phase, hipStream_t stream)
{
    const bool bf16 = a.dt == MDN_BF16;
    if (phase == BOTH && bf16 && !a.row_split && a.nseg >= 3 && a.T > 0) {
        const hipError_t err = mdn::launch_chunk_fused_seg(
            a.q, a.k, a.v, a.alpha, a.mu, a.eta, a.beta, a.S0, a.M0, a.O, a.S_T, a.M_T, a.B, a.T,
            a.H, a.Dk, a.Dv, a.nseg, const_cast<void*>(a.ws), stream);
        return err == hipSuccess ? MDN_OK : MDN_ERR_HIP;
    }
    if (phase == BOTH && bf16 && !a.row_split && a.T > 0) {
        const hipError_t err =
            mdn::launch_chunk_fused(a.q, a.k, a.v, a.alpha, a.mu, a.eta, a.beta, a.S0, a.M0, a.O,
                                    a.Vt, a.S_T, a.M_T, a.B, a.T, a.H, a.Dk, a.Dv,
                                    const_cast<void*>(a.ws), stream);
        return err == hipSuccess ? MDN_OK : MDN_ERR_HIP;
    }
    if ((phase & PREPARE) && a.T > 0) {
        const hipError_t err =
            mdn::launch_chunk_prepare(a.q, a.k, a.alpha, a.mu, a.eta, a.beta, a.B, a.T, a.H, a.Dk,
                                      bf16, const_cast<void*>(a.ws), stream);
        if (err != hipSuccess) return MDN_ERR_HIP;
    }
    if (phase & SCAN) {
        // a NULL mu (phase BOTH only: the scan entry point has no gates) means
        // mu = 0, and then M0 is not read
        const bool momentum = phase != BOTH || a.mu != nullptr;
        const float* M0 = momentum || a.T == 0 ? a.M0 : nullptr;
        const hipError_t err =
            mdn::launch_chunk_scan(a.q, a.k, a.v, a.S0, M0, a.O, a.Vt, a.S_T, a.M_T, a.B, a.T,
                                   a.H, a.Dk, a.Dv, bf16, a.row_split, momentum, a.ws, stream);
        if (err != hipSuccess) return MDN_ERR_HIP;
    }
    return MDN_OK;
}

mdn_status run_fwd(const FwdArgs& a, int phase, hipStream_t stream)
{
    bool no_work = false;
    const mdn_status st = validate_fwd(a, phase, &no_work);
    if (st != MDN_OK || no_work) return st;
    return launch_fwd(a, phase, stream);
}

// The forward's workspace for callers that cannot allocate: one array per
// device in the library's code object, loaded with it and held until the
// process ends.  In host code `scratch` names a host-side stand-in, not
// device memory; its device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is ever
// passed to a kernel.
static __device__ __align__(256) unsigned char scratch[MDN_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> scratch_ptr[MAX_DEVICES];
std::mutex scratch_mutex;

// The device address of `scratch` on the device `stream` belongs to (the
// current device for the null stream).
mdn_status scratch_for_stream(hipStream_t stream, void** out)
{
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return MDN_ERR_HIP;
    int dev = cur;
    if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return MDN_ERR_HIP;
    if (dev < 0 || dev >= MAX_DEVICES) return MDN_ERR_UNSUPPORTED;
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(scratch_mutex);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (dev != cur && hipSetDevice(dev) != hipSuccess) return MDN_ERR_HIP;
            const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (dev != cur && hipSetDevice(cur) != hipSuccess) return MDN_ERR_HIP;
            if (err != hipSuccess || p == nullptr) return MDN_ERR_HIP;
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MDN_OK;
}

}  // namespace

extern "C" {

mdn_status mdn_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                         const float* mu, const float* eta, const float* beta, const float* S0,
                         const float* M0, void* O, void* Vt, float* S_T, float* M_T, int B,
                         int T, int H, int Dk, int Dv, int chunk, mdn_dtype dt, void* workspace,
                         size_t workspace_bytes, hipStream_t stream)
{
    FwdArgs a{q, k, v, alpha, mu, eta, beta, S0, M0, O, Vt, S_T, M_T, B, T, H, Dk, Dv,
              chunk, dt, workspace, workspace_bytes};
    a.nseg = segments_for(B, T, H, Dk, Dv, dt, Vt != nullptr, mu != nullptr);
    a.row_split = a.nseg == 0 && row_split_for(B, H, Dv, dt, Vt != nullptr);
    return run_fwd(a, BOTH, stream);
}

mdn_status mdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const float* alpha, const float* mu, const float* eta,
                                 const float* beta, const float* S0, const float* M0, void* O,
                                 void* Vt, float* S_T, float* M_T, int B, int T, int H, int Dk,
                                 int Dv, int chunk, mdn_dtype dt, hipStream_t stream)
{
    FwdArgs a{q, k, v, alpha, mu, eta, beta, S0, M0, O, Vt, S_T, M_T, B, T, H, Dk, Dv,
              chunk, dt, nullptr, MDN_NOALLOC_SCRATCH_BYTES};
    a.static_ws = true;
    // the row split only where its workspace fits the array
    a.row_split = row_split_for(B, H, Dv, dt, Vt != nullptr) &&
                  split_workspace_bytes(B, T, H, Dk, Dv, chunk, dt) <= MDN_NOALLOC_SCRATCH_BYTES;
    bool no_work = false;
    mdn_status st = validate_fwd(a, BOTH, &no_work);
    if (st != MDN_OK || no_work) return st;
    if (split_workspace_bytes(B, T, H, Dk, Dv, chunk, dt) > 0) {
        void* p = nullptr;
        st = scratch_for_stream(stream, &p);
        if (st != MDN_OK) return st;
        a.ws = p;
    }
    return launch_fwd(a, BOTH, stream);
}

mdn_status mdn_chunk_fwd_prepare(const void* q, const void* k, const float* alpha,
                                 const float* mu, const float* eta, const float* beta, int B,
                                 int T, int H, int Dk, int chunk, mdn_dtype dt, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream)
{
    // the scan's Dv does not change the prepared data; any supported value
    // validates the same
    const FwdArgs a{q, k, nullptr, alpha, mu, eta, beta, nullptr, nullptr, nullptr, nullptr,
                    nullptr, nullptr, B, T, H, Dk, 64, chunk, dt, workspace, workspace_bytes};
    return run_fwd(a, PREPARE, stream);
}

mdn_status mdn_chunk_fwd_scan(const void* q, const void* k, const void* v, const float* S0,
                              const float* M0, void* O, float* S_T, float* M_T, int B, int T,
                              int H, int Dk, int Dv, int chunk, mdn_dtype dt,
                              const void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    FwdArgs a{q, k, v, nullptr, nullptr, nullptr, nullptr, S0, M0, O, nullptr, S_T, M_T, B,
              T, H, Dk, Dv, chunk, dt, workspace, workspace_bytes};
    a.row_split = row_split_for(B, H, Dv, dt, false);
    return run_fwd(a, SCAN, stream);
}

mdn_status mdn_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                           const float* mu, const float* eta, const float* beta, float* S,
                           float* M, void* o, int N, int H, int Dk, int Dv, mdn_dtype dt,
                           hipStream_t stream)
{
    if (N < 0 || H < 0) return MDN_ERR_SHAPE;
    if (!head_dim_ok(Dk) || !head_dim_ok(Dv)) return MDN_ERR_UNSUPPORTED;
    if (dt != MDN_F32 && dt != MDN_BF16) return MDN_ERR_UNSUPPORTED;
    if (N == 0 || H == 0) return MDN_OK;
    size_t heads, nstate;
    if (!mul_ok((size_t)N, (size_t)H, 1, 1, &heads) ||
        !mul_ok((size_t)N, (size_t)H, (size_t)Dk, (size_t)Dv, &nstate))
        return MDN_ERR_SHAPE;
    if (heads > 0x7fffffffu) return MDN_ERR_SHAPE;
    // mu may be NULL (mu = 0, the gated delta rule), and then M may be too
    if (!q || !k || !v || !alpha || !eta || !S || !o || (mu && !M)) return MDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, alpha, mu, eta, beta, S, M, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MDN_ERR_ALIGN;
    const size_t esz = dt == MDN_BF16 ? 2 : 4;
    const Span sq = span(q, heads * Dk * esz), sk = span(k, heads * Dk * esz),
               sv = span(v, heads * Dv * esz), sa = span(alpha, heads * 4),
               sm = span(mu, heads * 4), se = span(eta, heads * 4), sb = span(beta, heads * 4),
               sS = span(S, nstate * 4), sM = span(M, nstate * 4), so = span(o, heads * Dv * esz);
    const Span inputs[] = {sq, sk, sv, sa, sm, se, sb};
    for (const Span& x : inputs)
        if (overlap(so, x) || overlap(sS, x) || overlap(sM, x)) return MDN_ERR_ALIAS;
    if (overlap(so, sS) || overlap(so, sM) || overlap(sS, sM)) return MDN_ERR_ALIAS;
    const hipError_t err = mdn::launch_decode(q, k, v, alpha, mu, eta, beta, S, M, o, (int)heads,
                                              Dk, Dv, dt == MDN_BF16, stream);
    return err == hipSuccess ? MDN_OK : MDN_ERR_HIP;
}

mdn_status mdn_gates_from_logits(const float* z_eta, const float* z_alpha, const float* z_beta,
                                 const float* z_mu, size_t n, mdn_gate_params params,
                                 float* alpha, float* mu, float* eta, float* beta,
                                 hipStream_t stream)
{
    if (n == 0) return MDN_OK;
    const float* ins[] = {z_eta, z_alpha, z_beta, z_mu};
    float* outs[] = {alpha, mu, eta, beta};
    for (const float* p : ins)
        if (!p) return MDN_ERR_NULL;
    for (const float* p : outs)
        if (!p) return MDN_ERR_NULL;
    for (const float* p : ins)
        if (!aligned16(p)) return MDN_ERR_ALIGN;
    for (const float* p : outs)
        if (!aligned16(p)) return MDN_ERR_ALIGN;
    if (n > (size_t)-1 / 4) return MDN_ERR_SHAPE;
    const float pv[] = {params.tau, params.s, params.a, params.b, params.log_mu_min};
    for (float x : pv)
        if (!std::isfinite(x)) return MDN_ERR_UNSUPPORTED;
    if (!(params.tau > 0.f)) return MDN_ERR_UNSUPPORTED;
    Span sp[8];
    for (int i = 0; i < 4; ++i) {
        sp[i] = span(ins[i], n * 4);
        sp[4 + i] = span(outs[i], n * 4);
    }
    for (int i = 0; i < 8; ++i)
        for (int j = i + 1; j < 8; ++j)
            if ((i >= 4 || j >= 4) && overlap(sp[i], sp[j])) return MDN_ERR_ALIAS;
    const hipError_t err = mdn::launch_gates(z_eta, z_alpha, z_beta, z_mu, n, params.tau, params.s,
                                             params.a, params.b, params.log_mu_min, alpha, mu,
                                             eta, beta, stream);
    return err == hipSuccess ? MDN_OK : MDN_ERR_HIP;
}

size_t mdn_chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk,
                                     mdn_dtype dt)
{
    if (B <= 0 || T <= 0 || H <= 0) return 0;
    if (!head_dim_ok(Dk) || !head_dim_ok(Dv) || chunk != 64) return 0;
    if (dt != MDN_F32 && dt != MDN_BF16) return 0;
    size_t tmp;
    if (!mul_ok((size_t)B, (size_t)T, (size_t)H, 1, &tmp)) return 0;
    return mdn::chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, dt == MDN_BF16);
}

mdn_status mdn_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                         const float* mu, const float* eta, const float* beta, const float* S0,
                         const float* M0, const void* dO, const float* dS_T, const float* dM_T,
                         const void* Vt, float* dq, float* dk, float* dv, float* dalpha,
                         float* dmu, float* deta,
                         float* dbeta, float* dS0, float* dM0, int B, int T, int H, int Dk,
                         int Dv, int chunk, mdn_dtype dt, void* workspace,
                         size_t workspace_bytes, hipStream_t stream)
{
    if (B < 0 || T < 0 || H < 0) return MDN_ERR_SHAPE;
    if (!head_dim_ok(Dk) || !head_dim_ok(Dv) || chunk != 64) return MDN_ERR_UNSUPPORTED;
    if (dt != MDN_F32 && dt != MDN_BF16) return MDN_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return MDN_OK;
    const size_t esz = dt == MDN_BF16 ? 2 : 4;
    size_t nqk, nv, ngate, nstate;
    if (!mul_ok((size_t)B, (size_t)T, (size_t)H, (size_t)Dk, &nqk) ||
        !mul_ok((size_t)B, (size_t)T, (size_t)H, (size_t)Dv, &nv) ||
        !mul_ok((size_t)B, (size_t)T, (size_t)H, 1, &ngate) ||
        !mul_ok((size_t)B, (size_t)H, (size_t)Dk, (size_t)Dv, &nstate))
        return MDN_ERR_SHAPE;
    if ((size_t)B * H * (((size_t)T + 63) / 64) > 0xffffffffu) return MDN_ERR_SHAPE;
    const bool tok = T > 0;
    if (tok && (!q || !k || !v || !alpha || !eta || !dO || !dq || !dk || !dv || !dalpha || !deta))
        return MDN_ERR_NULL;
    const void* ptrs[] = {q, k, v, alpha, mu, eta, beta, S0, M0, dO, dS_T, dM_T, Vt, dq, dk, dv,
                          dalpha, dmu, deta, dbeta, dS0, dM0, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return MDN_ERR_ALIGN;
    const size_t need = tok ? mdn::chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, dt == MDN_BF16) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return MDN_ERR_WORKSPACE;

    const size_t nt = tok ? 1 : 0;
    // gradients of absent gates are not written
    float* dmu_w = mu ? dmu : nullptr;
    float* dbeta_w = beta ? dbeta : nullptr;
    const Span inputs[] = {span(q, nt * nqk * esz),     span(k, nt * nqk * esz),
                           span(v, nt * nv * esz),      span(alpha, nt * ngate * 4),
                           span(mu, nt * ngate * 4),    span(eta, nt * ngate * 4),
                           span(beta, nt * ngate * 4),  span(S0, nstate * 4),
                           span(M0, nstate * 4),        span(dO, nt * nv * esz),
                           span(dS_T, nstate * 4),      span(dM_T, nstate * 4),
                           span(Vt, nt * nv * esz)};
    const Span outputs[] = {span(dq, nt * nqk * 4),        span(dk, nt * nqk * 4),
                            span(dv, nt * nv * 4),         span(dalpha, nt * ngate * 4),
                            span(dmu_w, nt * ngate * 4),   span(deta, nt * ngate * 4),
                            span(dbeta_w, nt * ngate * 4), span(dS0, nstate * 4),
                            span(dM0, nstate * 4),         span(workspace, need)};
    constexpr int NO = sizeof(outputs) / sizeof(outputs[0]);
    for (int i = 0; i < NO; ++i) {
        for (const Span& x : inputs)
            if (overlap(outputs[i], x)) return MDN_ERR_ALIAS;
        for (int j = i + 1; j < NO; ++j)
            if (overlap(outputs[i], outputs[j])) return MDN_ERR_ALIAS;
    }

    if (!tok) {
        // no tokens: the state gradients pass straight through
        hipError_t err = hipSuccess;
        if (dS0) err = mdn::launch_state_copy(dS_T, dS0, nstate, stream);
        if (err == hipSuccess && dM0) err = mdn::launch_state_copy(dM_T, dM0, nstate, stream);
        return err == hipSuccess ? MDN_OK : MDN_ERR_HIP;
    }
    const hipError_t err = mdn::launch_chunk_bwd(
        q, k, v, alpha, mu, eta, beta, S0, M0, dO, dS_T, dM_T, Vt, dq, dk, dv, dalpha, dmu_w, deta,
        dbeta_w, dS0, dM0, B, T, H, Dk, Dv, dt == MDN_BF16, workspace, stream);
    return err == hipSuccess ? MDN_OK : MDN_ERR_HIP;
}

static mdn_status check_rows(size_t rows, int H, int D, mdn_dtype dt, float eps, size_t* bytes)
{
    if (H < 0) return MDN_ERR_SHAPE;
    if (!head_dim_ok(D)) return MDN_ERR_UNSUPPORTED;
    if (dt != MDN_F32 && dt != MDN_BF16) return MDN_ERR_UNSUPPORTED;
    if (!std::isfinite(eps) || !(eps > 0.f)) return MDN_ERR_UNSUPPORTED;
    size_t n;
    if (!mul_ok(rows, (size_t)H, (size_t)D, dt == MDN_BF16 ? 2 : 4, &n)) return MDN_ERR_SHAPE;
    *bytes = n;
    return MDN_OK;
}

// true when `out` overlaps none of `others`
static bool disjoint(const Span& out, std::initializer_list<Span> others)
{
    for (const Span& x : others)
        if (overlap(out, x)) return false;
    return true;
}

mdn_status mdn_qk_prologue(const void* q, const void* k, const float* d, void* q_out,
                           void* k_out, size_t rows, int H, int Dk, float eps, mdn_dtype dt,
                           hipStream_t stream)
{
    size_t bytes = 0;
    const mdn_status st = check_rows(rows, H, Dk, dt, eps, &bytes);
    if (st != MDN_OK) return st;
    if (bytes == 0) return MDN_OK;
    if (!q || !k || !q_out || !k_out) return MDN_ERR_NULL;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)d, (const void*)q_out,
                          (const void*)k_out})
        if (p && !aligned16(p)) return MDN_ERR_ALIGN;
    const Span sq = span(q, bytes), sk = span(k, bytes), sd = span(d, (size_t)H * 4),
               sqo = span(q_out, bytes), sko = span(k_out, bytes);
    // q_out may be q itself and k_out k itself; nothing else may overlap
    if (!(q_out == q ? disjoint(sqo, {sk, sd, sko}) : disjoint(sqo, {sq, sk, sd, sko})))
        return MDN_ERR_ALIAS;
    if (!(k_out == k ? disjoint(sko, {sq, sd}) : disjoint(sko, {sq, sk, sd})))
        return MDN_ERR_ALIAS;
    const hipError_t err = mdn::launch_qk_prologue(q, k, d, q_out, k_out, rows * (size_t)H, H,
                                                   Dk, dt == MDN_BF16, eps, stream);
    return err == hipSuccess ? MDN_OK : MDN_ERR_HIP;
}

mdn_status mdn_output_epilogue(const void* o, const void* g, const float* w, void* y,
                               size_t rows, int H, int Dv, float eps, mdn_dtype dt,
                               hipStream_t stream)
{
    size_t bytes = 0;
    const mdn_status st = check_rows(rows, H, Dv, dt, eps, &bytes);
    if (st != MDN_OK) return st;
    if (bytes == 0) return MDN_OK;
    if (!o || !g || !y) return MDN_ERR_NULL;
    for (const void* p : {(const void*)o, (const void*)g, (const void*)w, (const void*)y})
        if (p && !aligned16(p)) return MDN_ERR_ALIGN;
    const Span so = span(o, bytes), sg = span(g, bytes), sw = span(w, (size_t)Dv * 4),
               sy = span(y, bytes);
    // y may be o itself; nothing else may overlap it
    if (!(y == o ? disjoint(sy, {sg, sw}) : disjoint(sy, {so, sg, sw}))) return MDN_ERR_ALIAS;
    const hipError_t err = mdn::launch_output_epilogue(o, g, w, y, rows * (size_t)H, Dv,
                                                       dt == MDN_BF16, eps, stream);
    return err == hipSuccess ? MDN_OK : MDN_ERR_HIP;
}

}  // extern "C"
