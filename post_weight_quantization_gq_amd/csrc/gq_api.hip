// C ABI of libgq (declared in include/gq.h): argument validation, workspace
// handling and the launch sequences of the GuidedQuant Fisher and of LNQ.
#include "gq_common.h"
#include "gq_internal.h"
#include "gq.h"

static_assert((int)gq::ST_COUNT == (int)GQ_STAGE_COUNT, "stage ids of gq.h and the library differ");

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

// ---------------------------------------------------------------------------
// Per-stage HIP-event timing.  When enabled, every launch sequence of a stage is
// bracketed by two events recorded on the stream the kernels run on; reading
// synchronises the recorded events, sums their elapsed times per stage and
// returns the events to a pool.  A start mark is kept per (stage, stream), so
// timed calls on different streams pair their own events.
// ---------------------------------------------------------------------------
namespace gq {
namespace {
std::atomic<int> g_timing{0};      // bit mask of timed stages
std::mutex g_tmu;
struct Mark { int stage; hipEvent_t start, stop; };
std::vector<Mark> g_marks;          // completed (start, stop) pairs
std::vector<hipEvent_t> g_pool;     // reusable events
std::map<std::pair<int, hipStream_t>, hipEvent_t> g_open;   // start event of a stage in progress
bool g_err = false;                 // an event call failed since the last read

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

bool timing_on(Stage s) { return (g_timing.load(std::memory_order_relaxed) >> (int)s) & 1; }

hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, size_t> raised;
    std::lock_guard<std::mutex> lk(mu);
    size_t& have = raised[{kernel, dev}];
    if (bytes <= have) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) have = bytes;
    return e;
}

void timing_mark(Stage s, hipStream_t st, bool begin) {
    std::lock_guard<std::mutex> lk(g_tmu);
    const std::pair<int, hipStream_t> key{(int)s, st};
    auto it = g_open.find(key);
    hipEvent_t e = take_event();
    if (!e || hipEventRecord(e, st) != hipSuccess) {
        g_err = true;
        if (e) g_pool.push_back(e);
        if (!begin && it != g_open.end()) { g_pool.push_back(it->second); g_open.erase(it); }
        return;
    }
    if (begin) {
        if (it != g_open.end()) {
            g_pool.push_back(it->second);
            it->second = e;
        } else {
            g_open.emplace(key, e);
        }
    } else if (it != g_open.end()) {
        g_marks.push_back({(int)s, it->second, e});
        g_open.erase(it);
    } else {
        g_pool.push_back(e);
    }
}
}  // namespace gq

namespace {

thread_local std::string g_last_error;

gq_status fail(gq_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

gq_status hip_fail(hipError_t e, const char* where) {
    return fail(GQ_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool dtype_ok(gq_dtype t) { return t == GQ_F32 || t == GQ_BF16; }

// The kernels use 16-byte vector loads on X, G, W, F and P.
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workspace that is either the caller's or allocated stream-ordered for one call.
struct Scratch {
    void* ptr = nullptr;
    bool owned = false;
    hipStream_t st = nullptr;
    gq_status acquire(void* ws, size_t ws_bytes, size_t need, hipStream_t s) {
        st = s;
        if (ws) {
            if (ws_bytes < need)
                return fail(GQ_EINVAL, "workspace too small: %zu bytes given, %zu needed", ws_bytes,
                            need);
            ptr = ws;
            return GQ_OK;
        }
        if (need == 0) return GQ_OK;
        hipError_t e = hipMallocAsync(&ptr, need, s);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(GQ_ENOMEM, "hipMallocAsync(%zu) failed: %s", need, hipGetErrorString(e));
        }
        owned = true;
        return GQ_OK;
    }
    ~Scratch() {
        if (owned && ptr) (void)hipFreeAsync(ptr, st);
    }
};

gq_status check_lnq_shape(const float* F, int32_t groups, int64_t d_in, const void* W,
                          gq_dtype w_dt, int64_t d_out, int32_t bits, float ridge_rel) {
    if (!F || !W) return fail(GQ_EINVAL, "null F or W");
    if (!dtype_ok(w_dt)) return fail(GQ_EDTYPE, "unsupported W dtype %d", (int)w_dt);
    if (groups < 1) return fail(GQ_EINVAL, "groups must be >= 1 (got %d)", groups);
    if (d_out < 1 || d_in < 1) return fail(GQ_ESHAPE, "empty shape d_out=%lld d_in=%lld",
                                           (long long)d_out, (long long)d_in);
    if (d_out % groups) return fail(GQ_ESHAPE, "d_out=%lld is not a multiple of groups=%d",
                                    (long long)d_out, groups);
    if (d_in % 32) return fail(GQ_ESHAPE, "d_in=%lld must be a multiple of 32", (long long)d_in);
    if (d_in > 32768) return fail(GQ_ENOTIMPL, "d_in=%lld above 32768", (long long)d_in);
    if (bits < 1 || bits > 8) return fail(GQ_EINVAL, "bits=%d outside [1, 8]", bits);
    if (bits > 4)
        return fail(GQ_ENOTIMPL, "bits=%d: codebooks of more than 16 entries are not built "
                    "(the library takes 1..4 bits)", bits);
    if (!(ridge_rel >= 0.f) || !std::isfinite(ridge_rel))
        return fail(GQ_EINVAL, "ridge_rel must be finite and >= 0");
    if (!al16(F) || !al16(W)) return fail(GQ_EINVAL, "F and W must be 16-byte aligned");
    return GQ_OK;
}

bool block_ok(int32_t b) { return b == 64 || b == 128 || b == 256 || b == 512; }

int log2i(int32_t b) {
    int k = 0;
    while ((1 << k) < b) ++k;
    return k;
}

// Checked calls: copy a device flag to the host once the stream has reached it.
gq_status read_flag(const unsigned long long* dflag, hipStream_t st, unsigned long long* out) {
    hipError_t e = hipMemcpyAsync(out, dflag, sizeof(*out), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "checked call");
    return GQ_OK;
}

// NaN / Inf anywhere in W [d_out][d_in] or F [groups][d_in][d_in]: GQ_ENONFINITE, nothing
// written (the flag lives in the workspace).
gq_status check_lnq_inputs(const void* W, bool wb, int64_t d_out, int64_t d_in, const float* F,
                           int groups, unsigned long long* dflag, hipStream_t st) {
    hipError_t e = gq::lnq_zero_counter(dflag, 1, st);
    if (e == hipSuccess) e = gq::scan_nonfinite(W, wb, d_out * d_in, dflag, st);
    if (e == hipSuccess) e = gq::scan_nonfinite(F, false, (int64_t)groups * d_in * d_in, dflag, st);
    if (e != hipSuccess) return hip_fail(e, "finite check");
    unsigned long long bad = 0;
    gq_status rc = read_flag(dflag, st, &bad);
    if (rc != GQ_OK) return rc;
    if (bad) return fail(GQ_ENONFINITE, "W or F holds NaN or Inf; nothing was written");
    return GQ_OK;
}

bool ridge_ok(float r) { return r >= 0.f && std::isfinite(r); }

// Option checks shared by the whole-layer entry points.
gq_status check_options(const gq_lnq_options& o, int64_t d_in) {
    if (!ridge_ok(o.ridge_abs)) return fail(GQ_EINVAL, "ridge_abs must be finite and >= 0");
    if (o.check_finite != 0 && o.check_finite != 1) return fail(GQ_EINVAL, "check_finite must be 0 or 1");
    if (o.check_residual != 0 && o.check_residual != 1)
        return fail(GQ_EINVAL, "check_residual must be 0 or 1");
    if (!block_ok(o.block))
        return fail(GQ_EINVAL, "block=%d: the assignment block is 64, 128, 256 or 512", o.block);
    if (d_in % 64) return fail(GQ_ESHAPE, "d_in=%lld is not a multiple of 64", (long long)d_in);
    return GQ_OK;
}

}  // namespace

extern "C" {

int gq_abi_version(void) { return GQ_ABI_VERSION; }

void gq_timing_enable(int mask) { gq::g_timing.store(mask & ((1 << GQ_STAGE_COUNT) - 1)); }

gq_status gq_timing_read(double* ms, int64_t* launches) {
    if (!ms || !launches) return fail(GQ_EINVAL, "null ms or launches");
    std::lock_guard<std::mutex> lk(gq::g_tmu);
    for (int i = 0; i < GQ_STAGE_COUNT; ++i) { ms[i] = 0.0; launches[i] = 0; }
    gq_status rc = GQ_OK;
    if (gq::g_err) rc = fail(GQ_EHIP, "an event record failed while timing");
    for (const gq::Mark& m : gq::g_marks) {
        float t = 0.f;
        hipError_t e = hipEventSynchronize(m.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&t, m.start, m.stop);
        if (e != hipSuccess) {
            rc = hip_fail(e, "gq_timing_read");
        } else {
            ms[m.stage] += (double)t;
            launches[m.stage] += 1;
        }
        gq::g_pool.push_back(m.start);
        gq::g_pool.push_back(m.stop);
    }
    gq::g_marks.clear();
    gq::g_err = false;
    return rc;
}

const char* gq_stage_name(int stage) {
    static const char* names[GQ_STAGE_COUNT] = {
        "group_scale", "fisher_mfma", "fisher_finalize", "fisher_plain", "lnq_prepare",
        "lnq_resid", "lnq_init", "lnq_gram", "lnq_solve", "lnq_sweep", "lnq_small",
        "fisher_pack", "lnq_delta", "lut_pack", "lut_gemv", "fisher_h2d", "ganq_chol",
        "ganq_pass"};
    if (stage < 0 || stage >= GQ_STAGE_COUNT) return "";
    return names[stage];
}

const char* gq_last_error(void) { return g_last_error.c_str(); }

void gq_lnq_options_default(gq_lnq_options* opt) {
    if (!opt) return;
    opt->block = 512;
    opt->ridge_rel = 1e-6f;
    opt->init = GQ_INIT_QUANTILE;
    opt->gram_update = GQ_GRAM_AUTO;
    opt->ridge_abs = 0.f;
    opt->check_finite = 0;
    opt->check_residual = 0;
}

void lnq_options_default(lnq_options* opt) { gq_lnq_options_default(opt); }

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// The Fisher kernels' scratch, then one 256-byte slot for the flag of a checked call.
static size_t fisher_need(int64_t n, int64_t d_in, int32_t groups, bool bf16) {
    return al256(gq::fisher_workspace(n, d_in, groups, bf16)) + 256;
}

size_t gq_fisher_workspace_size(int64_t n, int64_t d_in, int64_t d_out, int32_t groups,
                                gq_dtype x_dt) {
    (void)d_out;
    if (n < 1 || d_in < 1 || groups < 1) return 0;
    return fisher_need(n, d_in, groups, x_dt == GQ_BF16);
}

gq_status gq_fisher_accumulate(const void* X, gq_dtype x_dt, int64_t n, int64_t d_in,
                               const void* G, gq_dtype g_dt, int64_t d_out, int32_t groups,
                               float* F, int32_t accumulate, void* ws, size_t ws_bytes,
                               void* stream) {
    if (!X || !G || !F) return fail(GQ_EINVAL, "null X, G or F");
    if (!dtype_ok(x_dt) || !dtype_ok(g_dt)) return fail(GQ_EDTYPE, "unsupported dtype");
    if (x_dt != g_dt) return fail(GQ_EDTYPE, "X and G must share a dtype");
    if (n < 1 || d_in < 1 || d_out < 1) return fail(GQ_ESHAPE, "empty shape");
    if (groups < 1) return fail(GQ_EINVAL, "groups must be >= 1");
    if (d_out % groups) return fail(GQ_ESHAPE, "d_out=%lld is not a multiple of groups=%d",
                                    (long long)d_out, groups);
    if (accumulate & ~(1 | GQ_FISHER_CHECK_FINITE))
        return fail(GQ_EINVAL, "accumulate must be 0 or 1, optionally | GQ_FISHER_CHECK_FINITE");
    if (!al16(X) || !al16(G) || !al16(F) || ((uintptr_t)ws & 255u))
        return fail(GQ_EINVAL, "X, G and F must be 16-byte aligned, ws 256-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    const bool bf16 = x_dt == GQ_BF16;
    const size_t need = fisher_need(n, d_in, groups, bf16);
    Scratch s;
    gq_status rc = s.acquire(ws, ws_bytes, need, st);
    if (rc != GQ_OK) return rc;
    hipError_t e;
    if (accumulate & GQ_FISHER_CHECK_FINITE) {
        unsigned long long* dflag = (unsigned long long*)((char*)s.ptr + need - 256);
        e = gq::lnq_zero_counter(dflag, 1, st);
        if (e == hipSuccess) e = gq::scan_nonfinite(X, bf16, n * d_in, dflag, st);
        if (e == hipSuccess) e = gq::scan_nonfinite(G, bf16, n * d_out, dflag, st);
        if (e != hipSuccess) return hip_fail(e, "finite check");
        unsigned long long bad = 0;
        if ((rc = read_flag(dflag, st, &bad)) != GQ_OK) return rc;
        if (bad) return fail(GQ_ENONFINITE, "X or G holds NaN or Inf; F was not written");
    }
    e = gq::fisher_run(X, G, bf16, n, d_in, d_out, groups, F, accumulate & 1, s.ptr, st);
    if (e != hipSuccess) return hip_fail(e, "gq_fisher_accumulate");
    return GQ_OK;
}

size_t gq_fisher_stream_workspace_size(int64_t chunk_tokens, int64_t d_in, int64_t d_out,
                                       int32_t groups, gq_dtype x_dt) {
    if (chunk_tokens < 1 || d_in < 1 || d_out < 1 || groups < 1 || !dtype_ok(x_dt)) return 0;
    const size_t es = x_dt == GQ_BF16 ? 2 : 4;
    return al256(gq::fisher_workspace(chunk_tokens, d_in, groups, x_dt == GQ_BF16)) +
           2 * al256((size_t)chunk_tokens * d_in * es) + 2 * al256((size_t)chunk_tokens * d_out * es);
}

// Host-resident X and G, streamed in chunks of T tokens.  Chunk k is copied on a copy
// stream into device buffer k % 2 while chunk k - 1's Fisher runs on `stream` and adds
// into F (the first chunk with the caller's `accumulate`).  Events order the buffers:
// chunk k's Fisher waits for its copy, chunk k + 2's copy waits for chunk k's Fisher,
// and the first copy waits for the work already on `stream` (which may still use ws).
gq_status gq_fisher_accumulate_host(const void* X, gq_dtype x_dt, int64_t n, int64_t d_in,
                                    const void* G, gq_dtype g_dt, int64_t d_out, int32_t groups,
                                    float* F, int32_t accumulate, int64_t chunk_tokens, void* ws,
                                    size_t ws_bytes, void* stream) {
    if (!X || !G || !F) return fail(GQ_EINVAL, "null X, G or F");
    if (!dtype_ok(x_dt) || !dtype_ok(g_dt)) return fail(GQ_EDTYPE, "unsupported dtype");
    if (x_dt != g_dt) return fail(GQ_EDTYPE, "X and G must share a dtype");
    if (n < 1 || d_in < 1 || d_out < 1) return fail(GQ_ESHAPE, "empty shape");
    if (groups < 1) return fail(GQ_EINVAL, "groups must be >= 1");
    if (d_out % groups) return fail(GQ_ESHAPE, "d_out=%lld is not a multiple of groups=%d",
                                    (long long)d_out, groups);
    if (accumulate != 0 && accumulate != 1) return fail(GQ_EINVAL, "accumulate must be 0 or 1");
    if (chunk_tokens < 1) return fail(GQ_EINVAL, "chunk_tokens must be >= 1");
    if (!al16(F) || ((uintptr_t)ws & 255u)) return fail(GQ_EINVAL, "F must be 16-byte and ws 256-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    const bool bf16 = x_dt == GQ_BF16;
    const int64_t T = chunk_tokens < n ? chunk_tokens : n;
    const size_t es = bf16 ? 2 : 4;
    const size_t fws = al256(gq::fisher_workspace(T, d_in, groups, bf16));
    const size_t xbytes = al256((size_t)T * d_in * es), gbytes = al256((size_t)T * d_out * es);
    Scratch s;
    gq_status rc = s.acquire(ws, ws_bytes, fws + 2 * xbytes + 2 * gbytes, st);
    if (rc != GQ_OK) return rc;
    char* base = (char*)s.ptr;
    void* xb[2] = {base + fws, base + fws + xbytes};
    void* gb[2] = {base + fws + 2 * xbytes, base + fws + 2 * xbytes + gbytes};

    hipStream_t cs = nullptr;
    hipEvent_t ev[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};   // copied x2, consumed x2, start
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    for (int i = 0; i < 5 && e == hipSuccess; ++i) e = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(ev[4], st);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs, ev[4], 0);
    const int64_t nchunks = (n + T - 1) / T;
    for (int64_t k = 0; k < nchunks && e == hipSuccess; ++k) {
        const int b = (int)(k & 1);
        const int64_t t0 = k * T;
        const int64_t tk = (n - t0) < T ? (n - t0) : T;
        if (k >= 2) e = hipStreamWaitEvent(cs, ev[2 + b], 0);
        if (e == hipSuccess) {
            gq::StageTimer tm(gq::ST_FISHER_H2D, cs);
            e = hipMemcpyAsync(xb[b], (const char*)X + (size_t)t0 * d_in * es, (size_t)tk * d_in * es,
                               hipMemcpyHostToDevice, cs);
            if (e == hipSuccess)
                e = hipMemcpyAsync(gb[b], (const char*)G + (size_t)t0 * d_out * es,
                                   (size_t)tk * d_out * es, hipMemcpyHostToDevice, cs);
        }
        if (e == hipSuccess) e = hipEventRecord(ev[b], cs);
        if (e == hipSuccess) e = hipStreamWaitEvent(st, ev[b], 0);
        if (e == hipSuccess)
            e = gq::fisher_run(xb[b], gb[b], bf16, tk, d_in, d_out, groups, F,
                               (k == 0) ? accumulate : 1, base, st);
        if (e == hipSuccess) e = hipEventRecord(ev[2 + b], st);
    }
    // the stream and events are released once their pending work completes
    for (int i = 0; i < 5; ++i)
        if (ev[i]) (void)hipEventDestroy(ev[i]);
    if (cs) (void)hipStreamDestroy(cs);
    if (e != hipSuccess) return hip_fail(e, "gq_fisher_accumulate_host");
    return GQ_OK;
}

size_t gq_lnq_workspace_size(int64_t d_out, int64_t d_in, int32_t groups, int32_t bits,
                             gq_dtype w_dt) {
    (void)w_dt;
    if (d_out < 1 || d_in < 1 || groups < 1 || bits < 1 || bits > 8) return 0;
    return gq::lnq_sizes(d_out, d_in, groups, 1 << bits).total;
}

size_t lnq_workspace_size(int64_t d_out, int64_t d_in, int32_t groups, int32_t bits,
                          gq_dtype w_dt) {
    return gq_lnq_workspace_size(d_out, d_in, groups, bits, w_dt);
}

gq_status lnq_codebook_update(const float* F, int32_t groups, int64_t d_in, const void* W,
                              gq_dtype w_dt, int64_t d_out, const uint8_t* P, int32_t bits,
                              float* C, float ridge_rel, int64_t* n_not_pd, void* ws,
                              size_t ws_bytes, void* stream) {
    gq_status rc = check_lnq_shape(F, groups, d_in, W, w_dt, d_out, bits, ridge_rel);
    if (rc != GQ_OK) return rc;
    if (!P || !C) return fail(GQ_EINVAL, "null P or C");
    if (!al16(P) || ((uintptr_t)ws & 255u)) return fail(GQ_EINVAL, "P must be 16-byte and ws 256-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    const bool wb = w_dt == GQ_BF16;
    const int m = 1 << bits;
    gq::LnqSizes z = gq::lnq_sizes(d_out, d_in, groups, m);
    Scratch s;
    if ((rc = s.acquire(ws, ws_bytes, z.total, st)) != GQ_OK) return rc;
    gq::LnqWs w = gq::lnq_carve(s.ptr, z);
    hipError_t e;
    if ((e = gq::lnq_prepare(F, groups, d_in, ridge_rel, 0.0, w, st)) != hipSuccess) return hip_fail(e, "prepare");
    if ((e = gq::lnq_codebook_step(F, W, wb, d_out, d_in, groups, m, P, C, w, w.objA,
                                   (unsigned long long*)n_not_pd, nullptr, st)) != hipSuccess)
        return hip_fail(e, "codebook");
    return GQ_OK;
}

gq_status lnq_assign_sweep(const float* F, int32_t groups, int64_t d_in, const void* W,
                           gq_dtype w_dt, int64_t d_out, const float* C, int32_t bits,
                           uint8_t* P, float ridge_rel, int32_t block, int64_t* n_changed,
                           void* ws, size_t ws_bytes, void* stream) {
    gq_status rc = check_lnq_shape(F, groups, d_in, W, w_dt, d_out, bits, ridge_rel);
    if (rc != GQ_OK) return rc;
    if (!P || !C) return fail(GQ_EINVAL, "null P or C");
    if (!al16(P) || ((uintptr_t)ws & 255u)) return fail(GQ_EINVAL, "P must be 16-byte and ws 256-byte aligned");
    if (!block_ok(block)) return fail(GQ_EINVAL, "block=%d: the assignment block is 64, 128, 256 or 512", block);
    if (d_in % 64) return fail(GQ_ESHAPE, "d_in=%lld is not a multiple of 64", (long long)d_in);
    hipStream_t st = (hipStream_t)stream;
    const bool wb = w_dt == GQ_BF16;
    const int m = 1 << bits;
    gq::LnqSizes z = gq::lnq_sizes(d_out, d_in, groups, m);
    Scratch s;
    if ((rc = s.acquire(ws, ws_bytes, z.total, st)) != GQ_OK) return rc;
    gq::LnqWs w = gq::lnq_carve(s.ptr, z);
    w.sb_shift = log2i(block);
    hipError_t e;
    if ((e = gq::lnq_prepare(F, groups, d_in, ridge_rel, 0.0, w, st)) != hipSuccess) return hip_fail(e, "prepare");
    if ((e = gq::lnq_sweep_step(F, W, wb, d_out, d_in, groups, C, m, P, w, w.objB, w.objC,
                                (unsigned long long*)n_changed, false, st)) != hipSuccess)
        return hip_fail(e, "sweep");
    return GQ_OK;
}

gq_status lnq_objective(const float* F, int32_t groups, int64_t d_in, const void* W,
                        gq_dtype w_dt, int64_t d_out, const float* C, const uint8_t* P,
                        int32_t bits, float ridge_rel, double* obj_rows, double* obj_total,
                        void* ws, size_t ws_bytes, void* stream) {
    gq_status rc = check_lnq_shape(F, groups, d_in, W, w_dt, d_out, bits, ridge_rel);
    if (rc != GQ_OK) return rc;
    if (!P || !C || !obj_rows) return fail(GQ_EINVAL, "null P, C or obj_rows");
    if (!al16(P) || ((uintptr_t)ws & 255u)) return fail(GQ_EINVAL, "P must be 16-byte and ws 256-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    const bool wb = w_dt == GQ_BF16;
    const int m = 1 << bits;
    gq::LnqSizes z = gq::lnq_sizes(d_out, d_in, groups, m);
    Scratch s;
    if ((rc = s.acquire(ws, ws_bytes, z.total, st)) != GQ_OK) return rc;
    gq::LnqWs w = gq::lnq_carve(s.ptr, z);
    hipError_t e;
    if ((e = gq::lnq_prepare(F, groups, d_in, ridge_rel, 0.0, w, st)) != hipSuccess) return hip_fail(e, "prepare");
    if ((e = gq::lnq_objective_rows(W, wb, d_out, d_in, groups, m, P, C, w, obj_rows, st)) != hipSuccess)
        return hip_fail(e, "objective");
    if (obj_total && (e = gq::lnq_reduce(obj_rows, d_out, obj_total, st)) != hipSuccess)
        return hip_fail(e, "objective sum");
    return GQ_OK;
}

}  // extern "C"

namespace {

// Debug check of the assignment passes (option check_residual): after a pass, every
// row's objective recomputed from scratch, with a residual array of its own, against
// the objective the pass reached through its running residual.  Its buffers are
// allocated stream-ordered for the call; the run itself is unchanged (the recomputation
// writes only its own residual, its own objectives and the error planes, which every
// residual product rewrites before reading).
constexpr double kPassCheckTol = 1e-4;   // relative to the row's objective at the pass start

struct PassCheck {
    Scratch s;
    float* R = nullptr;
    double* obj = nullptr;
    gq_status init(int64_t d_out, int64_t d_in, hipStream_t st) {
        const size_t rb = ((size_t)d_out * d_in * sizeof(float) + 255) & ~(size_t)255;
        gq_status rc = s.acquire(nullptr, 0, rb + (size_t)d_out * sizeof(double), st);
        if (rc != GQ_OK) return rc;
        R = (float*)s.ptr;
        obj = (double*)((char*)s.ptr + rb);
        return GQ_OK;
    }
    // w.objB / w.objC hold each row's objective at the pass start and the one it claims
    // at its end; mismatches are counted into w.cnt[9]
    hipError_t after_pass(const void* W, bool wb, int64_t d_out, int64_t d_in, int groups, int m,
                          const uint8_t* P, const float* C, const gq::LnqWs& w, hipStream_t st) {
        gq::LnqWs wd = w;
        wd.R = R;
        hipError_t e = gq::lnq_objective_rows(W, wb, d_out, d_in, groups, m, P, C, wd, obj, st);
        if (e != hipSuccess) return e;
        return gq::lnq_check_claim(w.objB, w.objC, obj, d_out, kPassCheckTol, w.cnt + 9, st);
    }
    gq_status verdict(const gq::LnqWs& w, hipStream_t st) {
        unsigned long long bad = 0;
        gq_status rc = read_flag(w.cnt + 9, st, &bad);
        if (rc != GQ_OK) return rc;
        if (bad)
            return fail(GQ_ECHECK, "%llu (row, pass) objectives reached through the running "
                        "residual differ from a fresh F'e by more than %g of the row's "
                        "objective", bad, kPassCheckTol);
        return GQ_OK;
    }
};

// Argument checks of lnq_quantize (before anything is enqueued).
gq_status lnq_quantize_check(const void* W, gq_dtype w_dt, int64_t d_out, int64_t d_in,
                             const float* F, int32_t groups, int32_t bits, int32_t iters,
                             const gq_lnq_options& o, const float* C, const uint8_t* P) {
    gq_status rc = check_lnq_shape(F, groups, d_in, W, w_dt, d_out, bits, o.ridge_rel);
    if (rc != GQ_OK) return rc;
    if (!P || !C) return fail(GQ_EINVAL, "null P or C");
    if (!al16(P)) return fail(GQ_EINVAL, "P must be 16-byte aligned");
    if (iters < 0) return fail(GQ_EINVAL, "iters must be >= 0");
    if (o.gram_update != GQ_GRAM_AUTO && o.gram_update != GQ_GRAM_DENSE)
        return fail(GQ_EINVAL, "unknown gram_update %d", o.gram_update);
    if (o.init != GQ_INIT_QUANTILE && o.init != GQ_INIT_GIVEN && o.init != GQ_INIT_UNIFORM)
        return fail(GQ_EINVAL, "unknown init %d", o.init);
    return check_options(o, d_in);
}

// The LNQ run of lnq_quantize on a workspace `base` of at least lnq_sizes().total bytes
// (arguments already checked).
gq_status lnq_quantize_run(const void* W, gq_dtype w_dt, int64_t d_out, int64_t d_in,
                           const float* F, int32_t groups, int32_t bits, int32_t iters,
                           const gq_lnq_options& o, float* C, uint8_t* P, double* obj_trace,
                           int64_t* n_changed, void* base, hipStream_t st) {
    gq_status rc;
    const bool wb = w_dt == GQ_BF16;
    const int m = 1 << bits;
    gq::LnqSizes z = gq::lnq_sizes(d_out, d_in, groups, m);
    gq::LnqWs w = gq::lnq_carve(base, z);
    w.sb_shift = log2i(o.block);
    if (o.check_finite && (rc = check_lnq_inputs(W, wb, d_out, d_in, F, groups, w.cnt + 8, st)) != GQ_OK)
        return rc;
    PassCheck pc;
    if (o.check_residual && (rc = pc.init(d_out, d_in, st)) != GQ_OK) return rc;
    hipError_t e;
    if ((e = gq::lnq_prepare(F, groups, d_in, o.ridge_rel, o.ridge_abs, w, st)) != hipSuccess)
        return hip_fail(e, "prepare");
    if (o.init == GQ_INIT_QUANTILE &&
        (e = gq::lnq_init_run(W, wb, d_out, d_in, m, C, P, st)) != hipSuccess)
        return hip_fail(e, "init");
    if (o.init == GQ_INIT_UNIFORM &&
        (e = gq::grid_init_run(W, wb, d_out, d_in, m, C, P, st)) != hipSuccess)
        return hip_fail(e, "init");
    // w.cnt: [0] moves of the pass, [1] rows not positive definite, [2] update mode,
    // [9] rows failing the pass check
    if ((e = gq::lnq_zero_counter(w.cnt, 3, st)) != hipSuccess) return hip_fail(e, "counter");
    if (o.check_residual && (e = gq::lnq_zero_counter(w.cnt + 9, 1, st)) != hipSuccess)
        return hip_fail(e, "counter");
    // A codebook step after a pass that changed at most incr_max codes updates A and the
    // residual from the changed coordinates (4 d bytes of F read per change, about
    // 3.5 ns per change at d = 4096) instead of recomputing them (2 d^2 d_out (m + 3)
    // matrix-core flops, about 1.7e-15 s per unit); the two costs meet near
    // 0.0017 d d_out (m + 3) changes.
    const bool incremental = o.gram_update == GQ_GRAM_AUTO;
    const int64_t incr_max = incremental ? d_out * d_in * (m + 3) * 17 / 10000 : -1;
    for (int t = 1; t <= iters; ++t) {
        // codebook step; objA = objective before it (trace entry 2t-2)
        if ((e = gq::lnq_codebook_step(F, W, wb, d_out, d_in, groups, m, P, C, w, w.objA,
                                       w.cnt + 1, incremental ? w.cnt + 2 : nullptr, st)) !=
            hipSuccess)
            return hip_fail(e, "codebook");
        // assignment pass; objB = objective after the codebook step (entry 2t-1), from
        // scratch; when recording, it also keeps the codes before it for the next step's
        // update
        if ((e = gq::lnq_sweep_step(F, W, wb, d_out, d_in, groups, C, m, P, w, w.objB,
                                    w.objC, w.cnt, incremental && t < iters, st)) != hipSuccess)
            return hip_fail(e, "sweep");
        if (o.check_residual &&
            (e = pc.after_pass(W, wb, d_out, d_in, groups, m, P, C, w, st)) != hipSuccess)
            return hip_fail(e, "pass check");
        // trace entries 2t-2 and 2t-1, the pass's move count, counter cleared, next mode
        if ((e = gq::lnq_iter_tail(w.objA, w.objB, d_out,
                                   obj_trace ? obj_trace + 2 * t - 2 : nullptr, w.cnt,
                                   n_changed ? n_changed + (t - 1) : nullptr, incr_max, st)) !=
            hipSuccess)
            return hip_fail(e, "iteration tail");
    }
    if (obj_trace) {
        // objective of the final (C, P), from scratch
        if ((e = gq::lnq_objective_rows(W, wb, d_out, d_in, groups, m, P, C, w, w.objA, st)) !=
            hipSuccess)
            return hip_fail(e, "final objective");
        if ((e = gq::lnq_reduce(w.objA, d_out, obj_trace + 2 * iters, st)) != hipSuccess)
            return hip_fail(e, "trace");
    }
    if (o.check_finite) {
        unsigned long long npd = 0;
        if ((rc = read_flag(w.cnt + 1, st, &npd)) != GQ_OK) return rc;
        if (npd)
            return fail(GQ_ENOTPD, "%llu codebook systems (rows x iterations) were not positive "
                        "definite; those rows kept their codebook", npd);
    }
    if (o.check_residual) return pc.verdict(w, st);
    return GQ_OK;
}

// ---------------------------------------------------------------------------
// The scratch of lnq_quantize_static: one array per device, of fixed size, held until
// the process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is taken once per device, with that device current, and
// only that address is used (kernel arguments, workspace carving).
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)GQ_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;     // device ordinal -> device address of `scratch`

gq_status static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *out = it->second;
        return GQ_OK;
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr.emplace(dev, ptr);
    *out = ptr;
    return GQ_OK;
}

}  // namespace

extern "C" {

gq_status lnq_quantize(const void* W, gq_dtype w_dt, int64_t d_out, int64_t d_in, const float* F,
                       int32_t groups, int32_t bits, int32_t iters, const gq_lnq_options* opt,
                       float* C, uint8_t* P, double* obj_trace, int64_t* n_changed, void* ws,
                       size_t ws_bytes, void* stream) {
    gq_lnq_options o;
    gq_lnq_options_default(&o);
    if (opt) o = *opt;
    gq_status rc = lnq_quantize_check(W, w_dt, d_out, d_in, F, groups, bits, iters, o, C, P);
    if (rc != GQ_OK) return rc;
    if ((uintptr_t)ws & 255u) return fail(GQ_EINVAL, "ws must be 256-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    Scratch s;
    if ((rc = s.acquire(ws, ws_bytes, gq::lnq_sizes(d_out, d_in, groups, 1 << bits).total, st)) !=
        GQ_OK)
        return rc;
    return lnq_quantize_run(W, w_dt, d_out, d_in, F, groups, bits, iters, o, C, P, obj_trace,
                            n_changed, s.ptr, st);
}

size_t lnq_static_scratch_bytes(void) { return kStaticScratchBytes; }

gq_status lnq_quantize_static(const void* W, gq_dtype w_dt, int64_t d_out, int64_t d_in,
                              const float* F, int32_t groups, int32_t bits, int32_t iters,
                              const gq_lnq_options* opt, float* C, uint8_t* P, double* obj_trace,
                              int64_t* n_changed, void* stream) {
    gq_lnq_options o;
    gq_lnq_options_default(&o);
    if (opt) o = *opt;
    gq_status rc = lnq_quantize_check(W, w_dt, d_out, d_in, F, groups, bits, iters, o, C, P);
    if (rc != GQ_OK) return rc;
    if (o.check_residual)
        return fail(GQ_EINVAL, "check_residual allocates its buffers; lnq_quantize_static "
                    "allocates nothing (use lnq_quantize)");
    const size_t need = gq::lnq_sizes(d_out, d_in, groups, 1 << bits).total;
    if (need > kStaticScratchBytes)
        return fail(GQ_ENOTIMPL, "this layer needs %zu bytes of scratch; lnq_quantize_static "
                    "holds %zu (use lnq_quantize with a workspace)", need, kStaticScratchBytes);
    void* base = nullptr;
    if ((rc = static_scratch(&base)) != GQ_OK) return rc;
    return lnq_quantize_run(W, w_dt, d_out, d_in, F, groups, bits, iters, o, C, P, obj_trace,
                            n_changed, base, (hipStream_t)stream);
}

gq_status grid_quantize(const void* W, gq_dtype w_dt, int64_t d_out, int64_t d_in, const float* F,
                        int32_t groups, int32_t bits, int32_t iters, const gq_lnq_options* opt,
                        float* C, uint8_t* P, double* obj_trace, int64_t* n_changed, void* ws,
                        size_t ws_bytes, void* stream) {
    gq_lnq_options o;
    gq_lnq_options_default(&o);
    o.init = GQ_INIT_UNIFORM;
    if (opt) o = *opt;
    gq_status rc = check_lnq_shape(F, groups, d_in, W, w_dt, d_out, bits, o.ridge_rel);
    if (rc != GQ_OK) return rc;
    if (!P || !C) return fail(GQ_EINVAL, "null P or C");
    if (!al16(P) || ((uintptr_t)ws & 255u)) return fail(GQ_EINVAL, "P must be 16-byte and ws 256-byte aligned");
    if (iters < 0) return fail(GQ_EINVAL, "iters must be >= 0");
    if (o.init != GQ_INIT_UNIFORM && o.init != GQ_INIT_GIVEN)
        return fail(GQ_EINVAL, "grid_quantize keeps a uniform grid: init must be UNIFORM or GIVEN, not %d",
                    o.init);
    if ((rc = check_options(o, d_in)) != GQ_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const bool wb = w_dt == GQ_BF16;
    const int m = 1 << bits;
    gq::LnqSizes z = gq::lnq_sizes(d_out, d_in, groups, m);
    Scratch s;
    if ((rc = s.acquire(ws, ws_bytes, z.total, st)) != GQ_OK) return rc;
    gq::LnqWs w = gq::lnq_carve(s.ptr, z);
    w.sb_shift = log2i(o.block);
    if (o.check_finite && (rc = check_lnq_inputs(W, wb, d_out, d_in, F, groups, w.cnt + 8, st)) != GQ_OK)
        return rc;
    PassCheck pc;
    if (o.check_residual && (rc = pc.init(d_out, d_in, st)) != GQ_OK) return rc;
    hipError_t e;
    if ((e = gq::lnq_prepare(F, groups, d_in, o.ridge_rel, o.ridge_abs, w, st)) != hipSuccess)
        return hip_fail(e, "prepare");
    if (o.init == GQ_INIT_UNIFORM &&
        (e = gq::grid_init_run(W, wb, d_out, d_in, m, C, P, st)) != hipSuccess)
        return hip_fail(e, "init");
    if (iters > 0 && (e = gq::lnq_zero_counter(w.cnt, 3, st)) != hipSuccess)
        return hip_fail(e, "counter");
    if (o.check_residual && (e = gq::lnq_zero_counter(w.cnt + 9, 1, st)) != hipSuccess)
        return hip_fail(e, "counter");
    for (int t = 1; t <= iters; ++t) {
        // assignment pass; objB = the objective before it, from the residual recomputed
        // from (C, P) at its start (trace entry t - 1)
        if ((e = gq::lnq_sweep_step(F, W, wb, d_out, d_in, groups, C, m, P, w, w.objB,
                                    w.objC, w.cnt, false, st)) != hipSuccess)
            return hip_fail(e, "sweep");
        if (o.check_residual &&
            (e = pc.after_pass(W, wb, d_out, d_in, groups, m, P, C, w, st)) != hipSuccess)
            return hip_fail(e, "pass check");
        if (obj_trace && (e = gq::lnq_reduce(w.objB, d_out, obj_trace + t - 1, st)) != hipSuccess)
            return hip_fail(e, "trace");
        // the pass's move count, counter cleared
        if ((e = gq::lnq_iter_tail(w.objA, w.objB, d_out, nullptr, w.cnt,
                                   n_changed ? n_changed + (t - 1) : nullptr, -1, st)) != hipSuccess)
            return hip_fail(e, "iteration tail");
    }
    if (obj_trace) {
        if ((e = gq::lnq_objective_rows(W, wb, d_out, d_in, groups, m, P, C, w, w.objA, st)) !=
            hipSuccess)
            return hip_fail(e, "final objective");
        if ((e = gq::lnq_reduce(w.objA, d_out, obj_trace + iters, st)) != hipSuccess)
            return hip_fail(e, "trace");
    }
    if (o.check_residual) return pc.verdict(w, st);
    return GQ_OK;
}

int64_t lut_packed_row_words(int64_t d_in, int32_t bits) {
    if (d_in < 1 || bits < 1 || bits > 4) return 0;
    return gq::lut_row_words(d_in, bits);
}

gq_status lut_pack_codes(const uint8_t* P, int64_t d_out, int64_t d_in, int32_t bits, uint32_t* Q,
                         void* stream) {
    if (!P || !Q) return fail(GQ_EINVAL, "null P or Q");
    if (d_out < 1 || d_in < 1) return fail(GQ_ESHAPE, "empty shape");
    if (bits < 1 || bits > 8) return fail(GQ_EINVAL, "bits=%d outside [1, 8]", bits);
    if (bits > 4) return fail(GQ_ENOTIMPL, "bits=%d: the packed layout takes 1..4", bits);
    if ((uintptr_t)Q & 15u) return fail(GQ_EINVAL, "Q must be 16-byte aligned");
    hipError_t e = gq::lut_pack_run(P, d_out, d_in, bits, Q, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "lut_pack_codes");
    return GQ_OK;
}

gq_status lut_gemv(const uint32_t* Q, const float* C, int64_t d_out, int64_t d_in, int32_t bits,
                   const void* x, gq_dtype x_dt, int32_t batch, float* y, void* stream) {
    if (!Q || !C || !x || !y) return fail(GQ_EINVAL, "null Q, C, x or y");
    if (!dtype_ok(x_dt)) return fail(GQ_EDTYPE, "unsupported dtype");
    if (d_out < 1 || d_in < 1) return fail(GQ_ESHAPE, "empty shape");
    if (bits < 1 || bits > 8) return fail(GQ_EINVAL, "bits=%d outside [1, 8]", bits);
    if (bits > 4) return fail(GQ_ENOTIMPL, "bits=%d: the packed layout takes 1..4", bits);
    if (batch < 1 || batch > 8) return fail(GQ_EINVAL, "batch=%d: 1..8 activation vectors", batch);
    if (((uintptr_t)Q & 15u) || ((uintptr_t)C & 3u) || ((uintptr_t)y & 3u) ||
        ((uintptr_t)x & (x_dt == GQ_BF16 ? 1u : 3u)))
        return fail(GQ_EINVAL, "Q must be 16-byte aligned, C, y and x element-aligned");
    const bool xb = x_dt == GQ_BF16;
    if (xb && !gq::lut_gemv_fits(d_in, bits, batch))
        return fail(GQ_ENOTIMPL, "d_in=%lld with batch=%d: one chunk of staged activations "
                    "exceeds the LDS", (long long)d_in, batch);
    hipError_t e = gq::lut_gemv_run(Q, C, d_out, d_in, bits, x, xb, batch, y, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "lut_gemv");
    return GQ_OK;
}

size_t ganq_workspace_size(int64_t d_out, int64_t d_in, int32_t groups, int32_t bits,
                           gq_dtype w_dt) {
    const size_t base = gq_lnq_workspace_size(d_out, d_in, groups, bits, w_dt);
    if (base == 0) return 0;
    return al256(base) + gq::ganq_extra_bytes(d_in, groups);
}

static gq_status ganq_setup(const float* F, int32_t groups, int64_t d_in, int64_t d_out,
                            int32_t bits, float ridge_rel, float ridge_abs, const void* W,
                            bool wb, bool check, void* ws, size_t ws_bytes, hipStream_t st,
                            Scratch& s, gq::LnqWs& w, gq::GanqWs& gw) {
    const int m = 1 << bits;
    gq::LnqSizes z = gq::lnq_sizes(d_out, d_in, groups, m);
    const size_t need = al256(z.total) + gq::ganq_extra_bytes(d_in, groups);
    gq_status rc = s.acquire(ws, ws_bytes, need, st);
    if (rc != GQ_OK) return rc;
    w = gq::lnq_carve(s.ptr, z);
    gw = gq::ganq_carve((char*)s.ptr + al256(z.total), d_in, groups);
    if (check && (rc = check_lnq_inputs(W, wb, d_out, d_in, F, groups, w.cnt + 8, st)) != GQ_OK)
        return rc;
    hipError_t e;
    if ((e = gq::lnq_prepare(F, groups, d_in, ridge_rel, ridge_abs, w, st)) != hipSuccess)
        return hip_fail(e, "prepare");
    if ((e = gq::ganq_factor(F, w.lam, d_in, groups, gw, st)) != hipSuccess) return hip_fail(e, "factor");
    return GQ_OK;
}

gq_status ganq_factor_damped(const float* F, int32_t groups, int64_t d_in, float ridge_rel,
                             float* L, int32_t* not_pd, void* ws, size_t ws_bytes, void* stream) {
    if (!F || !L) return fail(GQ_EINVAL, "null F or L");
    if (groups < 1 || d_in < 1) return fail(GQ_ESHAPE, "empty shape");
    if (d_in % 64) return fail(GQ_ESHAPE, "d_in=%lld is not a multiple of 64", (long long)d_in);
    if (!(ridge_rel >= 0.0f)) return fail(GQ_EINVAL, "ridge_rel must be >= 0");
    if (!al16(F) || !al16(L) || ((uintptr_t)ws & 255u)) return fail(GQ_EINVAL, "F, L 16-byte and ws 256-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    Scratch s;
    gq::LnqWs w;
    gq::GanqWs gw;
    // the factor needs no W-sized buffers: size them for one row
    gq_status rc = ganq_setup(F, groups, d_in, groups, 1, ridge_rel, 0.f, nullptr, false, false,
                              ws, ws_bytes, st, s, w, gw);
    if (rc != GQ_OK) return rc;
    hipError_t e = gq::ganq_factor_out(gw, d_in, groups, L, (int*)not_pd, st);
    if (e != hipSuccess) return hip_fail(e, "ganq_factor_damped");
    return GQ_OK;
}

gq_status ganq_quantize(const void* W, gq_dtype w_dt, int64_t d_out, int64_t d_in, const float* F,
                        int32_t groups, int32_t bits, int32_t iters, const gq_lnq_options* opt,
                        float* C, uint8_t* P, double* obj_trace, int64_t* n_changed,
                        int32_t* not_pd, void* ws, size_t ws_bytes, void* stream) {
    gq_lnq_options o;
    gq_lnq_options_default(&o);
    if (opt) o = *opt;
    gq_status rc = check_lnq_shape(F, groups, d_in, W, w_dt, d_out, bits, o.ridge_rel);
    if (rc != GQ_OK) return rc;
    if (!P || !C) return fail(GQ_EINVAL, "null P or C");
    if (!al16(P) || ((uintptr_t)ws & 255u)) return fail(GQ_EINVAL, "P must be 16-byte and ws 256-byte aligned");
    if (iters < 0) return fail(GQ_EINVAL, "iters must be >= 0");
    if (o.init != GQ_INIT_QUANTILE && o.init != GQ_INIT_GIVEN && o.init != GQ_INIT_UNIFORM)
        return fail(GQ_EINVAL, "unknown init %d", o.init);
    if ((rc = check_options(o, d_in)) != GQ_OK) return rc;
    if (o.check_residual)
        return fail(GQ_EINVAL, "check_residual checks the coordinate-descent pass's running "
                    "residual; the back-substitution pass keeps none");
    hipStream_t st = (hipStream_t)stream;
    const bool wb = w_dt == GQ_BF16;
    const int m = 1 << bits;
    Scratch s;
    gq::LnqWs w;
    gq::GanqWs gw;
    if ((rc = ganq_setup(F, groups, d_in, d_out, bits, o.ridge_rel, o.ridge_abs, W, wb,
                         o.check_finite != 0, ws, ws_bytes, st, s, w, gw)) != GQ_OK)
        return rc;
    hipError_t e;
    if (not_pd && (e = gq::ganq_factor_out(gw, d_in, groups, nullptr, (int*)not_pd, st)) != hipSuccess)
        return hip_fail(e, "factor flags");
    if (o.init == GQ_INIT_QUANTILE &&
        (e = gq::lnq_init_run(W, wb, d_out, d_in, m, C, P, st)) != hipSuccess)
        return hip_fail(e, "init");
    if (o.init == GQ_INIT_UNIFORM &&
        (e = gq::grid_init_run(W, wb, d_out, d_in, m, C, P, st)) != hipSuccess)
        return hip_fail(e, "init");
    if (iters > 0 && (e = gq::lnq_zero_counter(w.cnt, 3, st)) != hipSuccess)
        return hip_fail(e, "counter");
    for (int t = 1; t <= iters; ++t) {
        // codebook step (recomputed); objA = objective before it (trace entry 2t - 2)
        if ((e = gq::lnq_codebook_step(F, W, wb, d_out, d_in, groups, m, P, C, w, w.objA,
                                       w.cnt + 1, nullptr, st)) != hipSuccess)
            return hip_fail(e, "codebook");
        // objective after it (entry 2t - 1)
        if ((e = gq::lnq_objective_rows(W, wb, d_out, d_in, groups, m, P, C, w, w.objB, st)) !=
            hipSuccess)
            return hip_fail(e, "objective");
        // the back-substitution assignment; the residual buffer serves as its running sums
        if ((e = gq::ganq_assign_run(gw, d_in, d_out, groups, C, m, P, W, wb, w.R, w.cnt, st)) !=
            hipSuccess)
            return hip_fail(e, "assignment");
        if ((e = gq::lnq_iter_tail(w.objA, w.objB, d_out,
                                   obj_trace ? obj_trace + 2 * t - 2 : nullptr, w.cnt,
                                   n_changed ? n_changed + (t - 1) : nullptr, -1, st)) !=
            hipSuccess)
            return hip_fail(e, "iteration tail");
    }
    if (obj_trace) {
        if ((e = gq::lnq_objective_rows(W, wb, d_out, d_in, groups, m, P, C, w, w.objA, st)) !=
            hipSuccess)
            return hip_fail(e, "final objective");
        if ((e = gq::lnq_reduce(w.objA, d_out, obj_trace + 2 * iters, st)) != hipSuccess)
            return hip_fail(e, "trace");
    }
    if (o.check_finite) {
        std::vector<int> bad(groups, 0);
        e = hipMemcpyAsync(bad.data(), gw.bad, sizeof(int) * groups, hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e, "checked call");
        int nbad = 0;
        for (int b : bad) nbad += b != 0;
        if (nbad)
            return fail(GQ_ENOTPD, "%d groups' F' had a non-positive pivot; their rows kept their "
                        "codes", nbad);
    }
    return GQ_OK;
}

}  // extern "C"
