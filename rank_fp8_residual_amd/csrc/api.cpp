// C ABI of the fused LiteLinear forward (declared in include/litelinear.h):
// argument checks, the per-handle workspace, the choice between the skinny
// and the tiled kernels, and optional per-kernel event timing.
#include "litelinear.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <new>
#include <utility>
#include <vector>

#include "check.hpp"
#include "launch.hpp"

namespace {

constexpr int kNumKernels = 5;
// Largest M sent to the skinny kernel when the path is chosen automatically.
constexpr int64_t kSkinnyAutoMaxM = 64;

struct Prof {
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
    double total_ms = 0.0;
    int64_t launches = 0;
};

struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev) {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            changed = err == hipSuccess;
        }
    }
    ~DeviceGuard() {
        if (changed) (void)hipSetDevice(prev);
    }
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

using ll::aligned;
using ll::overlaps;

}  // namespace

// Workspace buffers of one call (device memory beyond the caller's tensors).
enum WsBuf {
    WS_APAD = 0,   // zero-padded copy of A [out, r_pad] (ranks not a multiple of 8, misaligned A)
    WS_APAD2,      // ... of a pair's second A
    WS_TWS,        // tiled: T' bf16 [M, r_pad]
    WS_TWS2,       // ... a pair's second T'
    WS_TPART,      // K-slice partial sums of T, float32 (both paths)
    WS_PARTIALS,   // skinny: K-slice partial sums of y, float32 [splits, M, out]
    WS_XQ,         // fp8-activation mode: e4m3fn codes of x [M, in]
    WS_XS,         // ... and the rows' scales [M]
    WS_SYNC,       // counters: zero before and after every launch
    WS_GEN,        // skinny all-of-K kernel: two 64-bit counters that only grow
                   // (zero when allocated or cleared after a failed wait)
    WS_COUNT
};

struct DevBuf {
    void *p = nullptr;
    size_t bytes = 0;
};

struct litelinear_ctx {
    int device = 0;
    DevBuf ws[WS_COUNT];
    DevBuf amax;                    // decomposition side: per-work-group max |R| (float bits)
    // Error word in host memory mapped into the device: kernels set it when
    // a bounded wait gives up.
    unsigned *err_host = nullptr;
    unsigned *err_dev = nullptr;
    bool sync_dirty = false;        // counters must be cleared before the next launch
    void *scratch = nullptr;        // the device's fixed scratch (litelinear_forward_noalloc)
    int64_t opt_path = 0, opt_out_f32 = 0, opt_split = 0, opt_profile = 0, opt_t_splits = 0, opt_t_launch = 0,
            opt_act_fp8 = 0, opt_gelu = 0, opt_test_wait = 0, opt_q_format = 0;
    Prof prof[kNumKernels];
    std::vector<hipEvent_t> event_pool;
};

namespace {

// True while `s` is being captured into a graph: no allocation, memset or
// event timing may be queued then.
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return st != hipStreamCaptureStatusNone;
}

// Grows a handle buffer to `need` bytes, stream-ordered on `s` (the old
// buffer is released once the stream's earlier work is done; nothing else on
// the device is waited for).  zero: the new memory is cleared on `s` before
// any later work of the stream uses it.
litelinear_status_t grow(DevBuf &b, size_t need, bool zero, hipStream_t s, bool in_capture) {
    if (b.bytes >= need) return LITELINEAR_OK;
    if (in_capture) return LITELINEAR_ERR_UNSUPPORTED;  // the workspace must be grown before capture
    const size_t bytes = (need + 255) & ~(size_t)255;
    if (b.p) {
        if (hipFreeAsync(b.p, s) != hipSuccess) return LITELINEAR_ERR_HIP;
        b.p = nullptr;
        b.bytes = 0;
    }
    if (hipMallocAsync(&b.p, bytes, s) != hipSuccess) {
        b.p = nullptr;
        (void)hipGetLastError();
        return LITELINEAR_ERR_OOM;
    }
    if (zero && ll::launch_fill_u32((unsigned *)b.p, (int64_t)(bytes / 4), 0u, s) != hipSuccess)
        return LITELINEAR_ERR_HIP;
    b.bytes = bytes;
    return LITELINEAR_OK;
}

hipEvent_t take_event(litelinear_ctx *h) {
    if (!h->event_pool.empty()) {
        hipEvent_t e = h->event_pool.back();
        h->event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launches `fn` on `s`, bracketed by an event pair when profiling is on
// (and the stream is not being captured).
template <class F>
litelinear_status_t timed_launch(litelinear_ctx *h, int kind, hipStream_t s, bool in_capture, F fn) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const bool prof = h->opt_profile && !in_capture;
    if (prof) {
        e0 = take_event(h);
        e1 = take_event(h);
        if (!e0 || !e1 || hipEventRecord(e0, s) != hipSuccess) return LITELINEAR_ERR_HIP;
    }
    if (fn() != hipSuccess) return LITELINEAR_ERR_HIP;
    if (prof) {
        if (hipEventRecord(e1, s) != hipSuccess) return LITELINEAR_ERR_HIP;
        h->prof[kind].pending.emplace_back(e0, e1);
    }
    return LITELINEAR_OK;
}

// A kernel reported a bounded wait that gave up: the status is returned
// once, and the counters are cleared before the next launch.
bool take_device_error(litelinear_ctx *h) {
    if (!h->err_host || __atomic_load_n(h->err_host, __ATOMIC_ACQUIRE) == 0) return false;
    __atomic_store_n(h->err_host, 0u, __ATOMIC_RELEASE);
    h->sync_dirty = true;
    return true;
}

}  // namespace

extern "C" {

const char *litelinear_version(void) { return "0.1.0"; }

const char *litelinear_status_string(litelinear_status_t s) {
    switch (s) {
        case LITELINEAR_OK: return "ok";
        case LITELINEAR_ERR_INVALID_ARG: return "invalid argument";
        case LITELINEAR_ERR_UNSUPPORTED: return "unsupported shape or alignment";
        case LITELINEAR_ERR_HIP: return "HIP runtime error";
        case LITELINEAR_ERR_OOM: return "out of device memory";
        case LITELINEAR_ERR_SYNC: return "a kernel's wait for other work-groups of its launch gave up (output undefined)";
        case LITELINEAR_ERR_SCRATCH: return "the call needs more workspace than the fixed no-allocation scratch holds";
    }
    return "unknown status";
}

litelinear_status_t litelinear_create(litelinear_handle_t *out, int device_ordinal) {
    if (!out) return LITELINEAR_ERR_INVALID_ARG;
    *out = nullptr;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess) {
        (void)hipGetLastError();
        return LITELINEAR_ERR_HIP;
    }
    if (device_ordinal < 0 || device_ordinal >= n) return LITELINEAR_ERR_INVALID_ARG;
    litelinear_ctx *h = new (std::nothrow) litelinear_ctx();
    if (!h) return LITELINEAR_ERR_OOM;
    h->device = device_ordinal;
    DeviceGuard g(h->device);
    void *dp = nullptr;
    if (g.err != hipSuccess ||
        hipHostMalloc((void **)&h->err_host, 64, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess ||
        hipHostGetDevicePointer(&dp, h->err_host, 0) != hipSuccess) {
        (void)hipGetLastError();
        if (h->err_host) (void)hipHostFree(h->err_host);
        delete h;
        return LITELINEAR_ERR_HIP;
    }
    *h->err_host = 0;
    h->err_dev = (unsigned *)dp;
    if (ll::scratch_init(h->device, &h->scratch) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipHostFree(h->err_host);
        delete h;
        return LITELINEAR_ERR_HIP;
    }
    *out = h;
    return LITELINEAR_OK;
}

litelinear_status_t litelinear_destroy(litelinear_handle_t h) {
    if (!h) return LITELINEAR_OK;
    litelinear_status_t st = LITELINEAR_OK;
    {
        DeviceGuard g(h->device);
        // The workspace came from stream-ordered allocations: released the
        // same way once the device is idle.
        if (hipDeviceSynchronize() != hipSuccess) st = LITELINEAR_ERR_HIP;
        for (DevBuf &b : h->ws)
            if (b.p) (void)hipFreeAsync(b.p, nullptr);
        if (h->amax.p) (void)hipFreeAsync(h->amax.p, nullptr);
        if (hipDeviceSynchronize() != hipSuccess) st = LITELINEAR_ERR_HIP;
        if (h->err_host) (void)hipHostFree(h->err_host);
        for (auto &p : h->prof)
            for (auto &e : p.pending) {
                (void)hipEventDestroy(e.first);
                (void)hipEventDestroy(e.second);
            }
        for (hipEvent_t e : h->event_pool) (void)hipEventDestroy(e);
    }
    delete h;
    return st;
}

litelinear_status_t litelinear_set_option(litelinear_handle_t h, int key, int64_t value) {
    if (!h) return LITELINEAR_ERR_INVALID_ARG;
    switch (key) {
        case LITELINEAR_OPT_PATH:
            if (value < 0 || value > 2) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_path = value;
            return LITELINEAR_OK;
        case LITELINEAR_OPT_OUTPUT_F32:
            if (value != 0 && value != 1) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_out_f32 = value;
            return LITELINEAR_OK;
        case LITELINEAR_OPT_SPLIT_K:
            if (value < 0 || value > 65535) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_split = value;
            return LITELINEAR_OK;
        case LITELINEAR_OPT_PROFILE:
            if (value != 0 && value != 1) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_profile = value;
            return LITELINEAR_OK;
        case LITELINEAR_OPT_T_SPLITS:
            if (value < 0 || value > 64) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_t_splits = value;
            return LITELINEAR_OK;
        case LITELINEAR_OPT_T_LAUNCH:
            if (value < 0 || value > 2) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_t_launch = value;
            return LITELINEAR_OK;
        case LITELINEAR_OPT_ACT_FP8:
            if (value != 0 && value != 1) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_act_fp8 = value;
            return LITELINEAR_OK;
        case LITELINEAR_OPT_ACTIVATION:
            if (value < 0 || value > 2) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_gelu = value;
            return LITELINEAR_OK;
        case LITELINEAR_OPT_Q_FORMAT:
            if (value != 0 && value != 1) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_q_format = value;
            return LITELINEAR_OK;
        case LITELINEAR_OPT_TEST_WAIT_TIMEOUT:
            if (value < 0 || value > (1 << 20)) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_test_wait = value;
            return LITELINEAR_OK;
    }
    return LITELINEAR_ERR_INVALID_ARG;
}

litelinear_status_t litelinear_kernel_time(litelinear_handle_t h, int kernel, double *total_ms,
                                           int64_t *launches, int reset) {
    if (!h || kernel < 0 || kernel >= kNumKernels) return LITELINEAR_ERR_INVALID_ARG;
    Prof &p = h->prof[kernel];
    litelinear_status_t st = LITELINEAR_OK;
    for (auto &e : p.pending) {
        float ms = 0.f;
        if (hipEventSynchronize(e.second) != hipSuccess || hipEventElapsedTime(&ms, e.first, e.second) != hipSuccess)
            st = LITELINEAR_ERR_HIP;
        p.total_ms += ms;
        p.launches += 1;
        h->event_pool.push_back(e.first);
        h->event_pool.push_back(e.second);
    }
    p.pending.clear();
    if (total_ms) *total_ms = p.total_ms;
    if (launches) *launches = p.launches;
    if (reset) {
        p.total_ms = 0.0;
        p.launches = 0;
    }
    return st;
}

litelinear_status_t litelinear_device_status(litelinear_handle_t h) {
    if (!h) return LITELINEAR_ERR_INVALID_ARG;
    return take_device_error(h) ? LITELINEAR_ERR_SYNC : LITELINEAR_OK;
}

}  // extern "C"

namespace {

// One output of a forward: y [M, out] = (x B^T) A^T + scale x dec(Q)^T + bias.
struct OutSet {
    const void *A, *Q, *bias;
    float scale;
    void *y;
    int64_t out;
};

// Polls before a bounded wait gives up (see the kernels): far beyond any
// real wait, which ends within microseconds.
constexpr unsigned kWaitLimit = 1u << 26;

// Where one call's workspace comes from: the handle's own buffers, grown on
// demand.  need[] holds each buffer's size for the call; take() returns the
// pointers, or a status.
struct WsRequest {
    size_t need[WS_COUNT] = {};
};

litelinear_status_t take_handle_ws(litelinear_ctx *h, const WsRequest &rq, hipStream_t s, bool in_capture,
                                   void *(&ptr)[WS_COUNT]) {
    for (int i = 0; i < WS_COUNT; ++i) {
        ptr[i] = nullptr;
        if (rq.need[i] == 0) continue;
        const litelinear_status_t st = grow(h->ws[i], rq.need[i], i == WS_SYNC || i == WS_GEN, s, in_capture);
        if (st != LITELINEAR_OK) return st;
        ptr[i] = h->ws[i].p;
    }
    return LITELINEAR_OK;
}

// The same request carved out of the device's fixed scratch (no
// allocation): the counters at its start, every other buffer after them on
// a 256-byte boundary.  SCRATCH when the call needs more than it holds.
litelinear_status_t take_scratch_ws(litelinear_ctx *h, const WsRequest &rq, void *(&ptr)[WS_COUNT]) {
    unsigned char *base = (unsigned char *)h->scratch;
    if (!base) return LITELINEAR_ERR_HIP;
    if (rq.need[WS_SYNC] > ll::kScratchSyncBytes) return LITELINEAR_ERR_SCRATCH;
    size_t off = ll::kScratchSyncBytes;
    for (int i = 0; i < WS_COUNT; ++i) {
        ptr[i] = nullptr;
        if (rq.need[i] == 0) continue;
        if (i == WS_SYNC) {
            ptr[i] = base;
            continue;
        }
        const size_t bytes = (rq.need[i] + 255) & ~(size_t)255;
        if (bytes > ll::kScratchBytes - off) return LITELINEAR_ERR_SCRATCH;
        ptr[i] = base + off;
        off += bytes;
    }
    return LITELINEAR_OK;
}

// The forward for one output, or for two sharing x and B (s2 != nullptr:
// the tiled kernel, T computed once).  Arguments are already checked.
// noalloc: the workspace comes from the device's fixed scratch, and the
// counters this call uses are cleared on the stream first.
litelinear_status_t forward_impl(litelinear_ctx *h, const void *x, int64_t ldx, const void *B, const OutSet &s1,
                                 const OutSet *s2, int64_t M, int64_t in, int64_t r, hipStream_t stream,
                                 bool noalloc = false) {
    const void *A = s1.A, *Q = s1.Q, *bias = s1.bias;
    void *y = s1.y;
    const float scale = s1.scale;
    const int64_t out = s1.out;
    const bool out_f32 = h->opt_out_f32 != 0;
    litelinear_status_t st = LITELINEAR_OK;
    if (take_device_error(h)) return LITELINEAR_ERR_SYNC;
    const bool in_capture = capturing(stream);
    // no event pairs under capture, nor in the no-allocation call (an event
    // is an allocation of its own)
    const bool no_events = in_capture || noalloc;
    const unsigned wait_limit = h->opt_test_wait > 0 ? (unsigned)h->opt_test_wait : kWaitLimit;
    const unsigned wait_extra = h->opt_test_wait > 0 ? 1u : 0u;

    const int64_t r_pad = r > 0 ? cdiv(r, 64) * 64 : 0;
    // The fp8-activation mode runs on the tiled kernel only (with in == 0
    // there is no residual product to run in fp8), and takes e4m3fn codes.
    const bool act8 = h->opt_act_fp8 != 0 && in > 0;
    const int q_format = (int)h->opt_q_format;
    const bool glu = h->opt_gelu == 2;
    if (act8 && q_format != 0) return LITELINEAR_ERR_UNSUPPORTED;
    if (glu && (s2 || out % 2 != 0)) return LITELINEAR_ERR_UNSUPPORTED;
    int64_t path = h->opt_path;
    ll::SkinnyPlan plan{};
    // (with the gated epilogue the skinny kernel reads Q, A and the partial
    // sums through whole-tensor descriptors, each below 2^31 bytes)
    const int64_t lim31 = (int64_t)1 << 31;
    const bool skinny_ok =
        !act8 && in > 0 && ll::skinny_supports(M) &&
        ll::skinny_shape_ok(M, in, out, r_pad, plan = ll::skinny_plan(M, in, out, r_pad, h->opt_split, glu), ldx) &&
        (!glu || (out * in < lim31 && out * (r_pad > 0 ? r_pad : 1) * 2 < lim31 &&
                  (int64_t)plan.splits * M * plan.tiles_n * 128 * 4 < lim31));
    if (s2) path = 2;
    if (path == 0) path = (M <= kSkinnyAutoMaxM && skinny_ok && !ll::tiled_tiny_shape(M, in, out, r)) ? 1 : 2;
    if (path == 1 && !skinny_ok) return LITELINEAR_ERR_UNSUPPORTED;

    // Workspace of this call.  A whose rows are not whole 16-byte chunks is
    // first copied into a zero-padded [out, r_pad] buffer (both paths read A
    // in 16-byte chunks).
    WsRequest rq;
    const bool pad1 = ll::a_needs_padding(r, A), pad2 = s2 && ll::a_needs_padding(r, s2->A);
    if (pad1) rq.need[WS_APAD] = (size_t)out * r_pad * 2;
    if (pad2) rq.need[WS_APAD2] = (size_t)s2->out * r_pad * 2;

    ll::SkinnyProblem sp{};
    ll::TiledProblem p{};
    ll::TileCfg mc{};
    bool producers = false;
    if (path == 1) {
        sp.plan = plan;
        // partial sums' rows: the products' columns (whole column tiles with
        // the gated epilogue)
        const int64_t pcols = glu ? (int64_t)plan.tiles_n * 128 : out;
        if (plan.splits > 1) rq.need[WS_PARTIALS] = (size_t)plan.splits * M * pcols * sizeof(float);
        if (r > 0) rq.need[WS_TPART] = (size_t)plan.t_splits * M * r_pad * sizeof(float);
        rq.need[WS_SYNC] = (size_t)ll::skinny_sync_words(plan) * sizeof(unsigned);
        // (the piece count and 32 ticket counters, 256 bytes apart)
        if (plan.fullk && r > 0) rq.need[WS_GEN] = 33 * 256;
    } else {
        p.x = x;
        p.ldx = ldx;
        p.A = A;
        p.B = B;
        p.Q = Q;
        p.bias = bias;
        p.y = y;
        p.scale = scale;
        p.M = M;
        p.K = in;
        p.N = out;
        p.r = r;
        p.r_pad = r_pad;
        p.out_f32 = out_f32;
        p.gelu = h->opt_gelu == 1;
        p.glu = glu;
        p.q_format = q_format;
        p.act8 = act8;
        if (s2) {
            p.Q2 = s2->Q;
            p.A2 = s2->A;
            p.bias2 = s2->bias;
            p.y2 = s2->y;
            p.scale2 = s2->scale;
            p.N2 = s2->out;
        }
        mc = ll::choose_main_tile(p);
        if (!ll::tiled_shape_ok(p, mc)) return LITELINEAR_ERR_UNSUPPORTED;
        if (act8) {
            rq.need[WS_XQ] = (size_t)M * in;
            rq.need[WS_XS] = (size_t)M * sizeof(float);
        }
        // With producers, T goes through the T' workspace and the row tiles'
        // ready counters; small problems compute it in each output tile instead.
        producers = r > 0 && !ll::tiled_self_t(p, mc);
        if (producers) {
            rq.need[WS_TWS] = (size_t)M * r_pad * 2;
            if (s2) rq.need[WS_TWS2] = (size_t)M * r_pad * 2;
            p.t_launch = ll::tiled_t_launch(p, mc, h->opt_t_launch);
            p.t_splits = p.t_launch > 0 ? 1 : ll::tiled_t_splits(p, mc, h->opt_t_splits);
            const int parts = p.t_launch > 0 ? p.t_launch : p.t_splits;
            if (parts > 1) rq.need[WS_TPART] = (size_t)parts * M * r_pad * sizeof(float);
            rq.need[WS_SYNC] = (size_t)ll::tiled_sync_words(p, mc) * sizeof(unsigned);
        }
    }

    void *ws[WS_COUNT];
    st = noalloc ? take_scratch_ws(h, rq, ws) : take_handle_ws(h, rq, stream, in_capture, ws);
    if (st != LITELINEAR_OK) return st;
    if (noalloc) {
        // The scratch is shared by every call on the device: its counters
        // are cleared for this call (a kernel, never a memset node).
        for (int i : {(int)WS_SYNC, (int)WS_GEN})
            if (rq.need[i] && ll::launch_fill_u32((unsigned *)ws[i], (int64_t)(rq.need[i] / 4), 0u, stream) !=
                                  hipSuccess)
                return LITELINEAR_ERR_HIP;
    } else if (h->sync_dirty) {
        // After a wait that gave up the counters may hold stale counts.
        for (int i : {(int)WS_SYNC, (int)WS_GEN})
            if (h->ws[i].p &&
                ll::launch_fill_u32((unsigned *)h->ws[i].p, (int64_t)(h->ws[i].bytes / 4), 0u, stream) != hipSuccess)
                return LITELINEAR_ERR_HIP;
        h->sync_dirty = false;
    }

    const void *a_eff = A;
    if (pad1) {
        st = timed_launch(h, LITELINEAR_KERNEL_PAD_A, stream, no_events,
                          [&] { return ll::launch_pad_a(A, ws[WS_APAD], out, r, r_pad, stream); });
        if (st != LITELINEAR_OK) return st;
        a_eff = ws[WS_APAD];
    }
    const void *a_eff2 = s2 ? s2->A : nullptr;
    if (pad2) {
        st = timed_launch(h, LITELINEAR_KERNEL_PAD_A, stream, no_events,
                          [&] { return ll::launch_pad_a(s2->A, ws[WS_APAD2], s2->out, r, r_pad, stream); });
        if (st != LITELINEAR_OK) return st;
        a_eff2 = ws[WS_APAD2];
    }

    if (path == 1) {
        sp.x = x;
        sp.ldx = ldx;
        sp.A = A;
        sp.B = B;
        sp.Q = Q;
        sp.bias = bias;
        sp.y = y;
        sp.scale = scale;
        sp.M = M;
        sp.K = in;
        sp.N = out;
        sp.r = r;
        sp.r_pad = r_pad;
        sp.out_f32 = out_f32;
        sp.gelu = h->opt_gelu == 1;
        sp.glu = glu;
        sp.q_format = q_format;
        sp.partials = (float *)ws[WS_PARTIALS];
        sp.t_part = (float *)ws[WS_TPART];
        sp.sync = (unsigned *)ws[WS_SYNC];
        sp.gen = (unsigned long long *)ws[WS_GEN];
        sp.err = h->err_dev;
        sp.wait_limit = wait_limit;
        sp.wait_extra = wait_extra;
        return timed_launch(h, LITELINEAR_KERNEL_SKINNY, stream, no_events,
                            [&] { return ll::launch_skinny(sp, a_eff, stream); });
    }

    if (act8) {
        p.xq = ws[WS_XQ];
        p.xs = (float *)ws[WS_XS];
        st = timed_launch(h, LITELINEAR_KERNEL_QUANT, stream, no_events,
                          [&] { return ll::launch_quant_rows(x, ldx, ws[WS_XQ], (float *)ws[WS_XS], M, in, stream); });
        if (st != LITELINEAR_OK) return st;
    }
    p.t_ws = ws[WS_TWS];
    p.t_ws2 = ws[WS_TWS2];
    p.t_part = (float *)ws[WS_TPART];
    p.err = h->err_dev;
    p.wait_limit = wait_limit;
    p.wait_extra = wait_extra;
    unsigned *sync = producers ? (unsigned *)ws[WS_SYNC] : nullptr;
    return timed_launch(h, LITELINEAR_KERNEL_MAIN, stream, no_events,
                        [&] { return ll::launch_tiled(p, mc, a_eff, a_eff2, sync, stream); });
}

}  // namespace

extern "C" {

litelinear_status_t litelinear_forward_strided(litelinear_handle_t h, const void *x, int64_t ldx, const void *A,
                                               const void *B, const void *Q, float scale, const void *bias, void *y,
                                               int64_t M, int64_t in, int64_t out, int64_t r, hipStream_t stream) {
    if (!h) return LITELINEAR_ERR_INVALID_ARG;
    const bool out_f32 = h->opt_out_f32 != 0;
    litelinear_status_t st = ll::check_args_ld(x, ldx, A, B, Q, bias, y, M, in, out, r, out_f32 ? 4 : 2, h->opt_gelu == 2);
    if (st != LITELINEAR_OK) return st;
    if (M == 0 || out == 0) return LITELINEAR_OK;
    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return LITELINEAR_ERR_HIP;
    return forward_impl(h, x, ldx, B, OutSet{A, Q, bias, scale, y, out}, nullptr, M, in, r, stream);
}

litelinear_status_t litelinear_forward(litelinear_handle_t h, const void *x, const void *A, const void *B,
                                       const void *Q, float scale, const void *bias, void *y, int64_t M,
                                       int64_t in, int64_t out, int64_t r, hipStream_t stream) {
    return litelinear_forward_strided(h, x, in, A, B, Q, scale, bias, y, M, in, out, r, stream);
}

litelinear_status_t litelinear_forward_noalloc(litelinear_handle_t h, const void *x, const void *A, const void *B,
                                               const void *Q, float scale, const void *bias, void *y, int64_t M,
                                               int64_t in, int64_t out, int64_t r, hipStream_t stream) {
    if (!h) return LITELINEAR_ERR_INVALID_ARG;
    litelinear_status_t st =
        ll::check_args_ld(x, in, A, B, Q, bias, y, M, in, out, r, h->opt_out_f32 != 0 ? 4 : 2, h->opt_gelu == 2);
    if (st != LITELINEAR_OK) return st;
    if (M == 0 || out == 0) return LITELINEAR_OK;
    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return LITELINEAR_ERR_HIP;
    return forward_impl(h, x, in, B, OutSet{A, Q, bias, scale, y, out}, nullptr, M, in, r, stream, true);
}

litelinear_status_t litelinear_forward_pair(litelinear_handle_t h, const void *x, const void *B, const void *A1,
                                            const void *Q1, float scale1, const void *bias1, void *y1, int64_t out1,
                                            const void *A2, const void *Q2, float scale2, const void *bias2, void *y2,
                                            int64_t out2, int64_t M, int64_t in, int64_t r, hipStream_t stream) {
    if (!h) return LITELINEAR_ERR_INVALID_ARG;
    if (h->opt_gelu == 2) return LITELINEAR_ERR_UNSUPPORTED;  // the gated epilogue has one output
    const int ysz = h->opt_out_f32 != 0 ? 4 : 2;
    litelinear_status_t st = litelinear_check_args(x, A1, B, Q1, bias1, y1, M, in, out1, r, ysz);
    if (st != LITELINEAR_OK) return st;
    st = litelinear_check_args(x, A2, B, Q2, bias2, y2, M, in, out2, r, ysz);
    if (st != LITELINEAR_OK) return st;
    // Each y must also stay clear of the other output's tensors.
    const uint64_t ny1 = (uint64_t)M * (uint64_t)out1 * ysz, ny2 = (uint64_t)M * (uint64_t)out2 * ysz;
    if (overlaps(y1, ny1, y2, ny2) || overlaps(y1, ny1, Q2, (uint64_t)out2 * in) ||
        overlaps(y1, ny1, bias2, (uint64_t)out2 * 2) || overlaps(y2, ny2, Q1, (uint64_t)out1 * in) ||
        overlaps(y2, ny2, bias1, (uint64_t)out1 * 2) ||
        (r > 0 && (overlaps(y1, ny1, A2, (uint64_t)out2 * r * 2) || overlaps(y2, ny2, A1, (uint64_t)out1 * r * 2))))
        return LITELINEAR_ERR_INVALID_ARG;
    if (M == 0 || (out1 == 0 && out2 == 0)) return LITELINEAR_OK;
    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return LITELINEAR_ERR_HIP;
    const OutSet s1{A1, Q1, bias1, scale1, y1, out1}, s2{A2, Q2, bias2, scale2, y2, out2};
    // One output empty, or the skinny regime (where T is a small part of
    // the time): one forward per output.  Otherwise one tiled launch.
    const bool skinny =
        h->opt_path == 1 || (h->opt_path == 0 && M <= kSkinnyAutoMaxM && h->opt_act_fp8 == 0);
    if (out1 == 0 || out2 == 0 || in == 0 || skinny) {
        if (out1 > 0 && (st = forward_impl(h, x, in, B, s1, nullptr, M, in, r, stream)) != LITELINEAR_OK) return st;
        if (out2 > 0) st = forward_impl(h, x, in, B, s2, nullptr, M, in, r, stream);
        return st;
    }
    return forward_impl(h, x, in, B, s1, &s2, M, in, r, stream);
}

litelinear_status_t litelinear_quantize_rows(litelinear_handle_t h, const void *x, int64_t M, int64_t in,
                                             void *codes, float *scales, hipStream_t stream) {
    if (!h || M < 0 || in < 0 || M > ((int64_t)1 << 40) || in > ((int64_t)1 << 40)) return LITELINEAR_ERR_INVALID_ARG;
    if ((double)M * (double)in > 4.0e18) return LITELINEAR_ERR_INVALID_ARG;
    if (M == 0) return LITELINEAR_OK;
    if (!scales || (in > 0 && (!x || !codes))) return LITELINEAR_ERR_INVALID_ARG;
    if (in % 16 != 0) return LITELINEAR_ERR_UNSUPPORTED;
    if ((in > 0 && (!aligned(x, 16) || !aligned(codes, 8))) || !aligned(scales, 4)) return LITELINEAR_ERR_UNSUPPORTED;
    if (in * 2 >= ((int64_t)1 << 31) || M >= ((int64_t)1 << 31)) return LITELINEAR_ERR_UNSUPPORTED;
    const uint64_t nx = (uint64_t)M * in * 2, nc = (uint64_t)M * in, ns = (uint64_t)M * 4;
    if (overlaps(codes, nc, x, nx) || overlaps(scales, ns, x, nx) || overlaps(scales, ns, codes, nc))
        return LITELINEAR_ERR_INVALID_ARG;
    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return LITELINEAR_ERR_HIP;
    return timed_launch(h, LITELINEAR_KERNEL_QUANT, stream, capturing(stream),
                        [&] { return ll::launch_quant_rows(x, in, codes, scales, M, in, stream); });
}

litelinear_status_t litelinear_quantize_tensor(litelinear_handle_t h, const float *R, int64_t n, void *codes,
                                               float *scale_out, hipStream_t stream) {
    if (!h || n < 0 || n > ((int64_t)1 << 40)) return LITELINEAR_ERR_INVALID_ARG;
    if (!scale_out || (n > 0 && (!R || !codes))) return LITELINEAR_ERR_INVALID_ARG;
    if (n % 4 != 0) return LITELINEAR_ERR_UNSUPPORTED;
    if ((n > 0 && (!aligned(R, 16) || !aligned(codes, 4))) || !aligned(scale_out, 4)) return LITELINEAR_ERR_UNSUPPORTED;
    if (n * 4 >= ((int64_t)1 << 31)) return LITELINEAR_ERR_UNSUPPORTED;
    if (overlaps(codes, (uint64_t)n, R, (uint64_t)n * 4) || overlaps(scale_out, 4, R, (uint64_t)n * 4) ||
        overlaps(scale_out, 4, codes, (uint64_t)n))
        return LITELINEAR_ERR_INVALID_ARG;
    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return LITELINEAR_ERR_HIP;
    const bool in_capture = capturing(stream);
    litelinear_status_t st = grow(h->amax, (size_t)ll::quant_tensor_slots(n) * 4, false, stream, in_capture);
    if (st != LITELINEAR_OK) return st;
    if (n == 0) {
        const float one = 1.0f;  // scale of an empty (all-zero) tensor
        return hipMemcpyAsync(scale_out, &one, 4, hipMemcpyHostToDevice, stream) == hipSuccess &&
                       hipStreamSynchronize(stream) == hipSuccess
                   ? LITELINEAR_OK
                   : LITELINEAR_ERR_HIP;
    }
    return timed_launch(h, LITELINEAR_KERNEL_CONVERT, stream, in_capture, [&] {
        return ll::launch_quant_tensor(R, n, codes, (unsigned *)h->amax.p, scale_out, stream);
    });
}

litelinear_status_t litelinear_residual_quantize(litelinear_handle_t h, const void *W, const void *A, const void *B,
                                                 int64_t out, int64_t in, int64_t r, void *codes, float *scale_out,
                                                 hipStream_t stream) {
    const int64_t lim = (int64_t)1 << 40;
    if (!h || out < 0 || in < 0 || r < 0 || out > lim || in > lim || r > lim) return LITELINEAR_ERR_INVALID_ARG;
    if ((double)out * (double)in > 4.0e18 || (double)r * (double)(in + out) > 4.0e18) return LITELINEAR_ERR_INVALID_ARG;
    if (!scale_out) return LITELINEAR_ERR_INVALID_ARG;
    if (out > 0 && in > 0 && (!W || !codes || (r > 0 && (!A || !B)))) return LITELINEAR_ERR_INVALID_ARG;
    if (in % 16 != 0 || r % 8 != 0) return LITELINEAR_ERR_UNSUPPORTED;
    if (!aligned(scale_out, 4) || (out > 0 && in > 0 && (!aligned(W, 16) || !aligned(codes, 16))) ||
        (r > 0 && out > 0 && in > 0 && (!aligned(A, 16) || !aligned(B, 16))))
        return LITELINEAR_ERR_UNSUPPORTED;
    const int64_t l31 = (int64_t)1 << 31;
    if (out * in * 2 >= l31 || out * r * 2 >= l31 || r * in * 2 >= l31) return LITELINEAR_ERR_UNSUPPORTED;
    const uint64_t nc = (uint64_t)out * in;
    if (overlaps(codes, nc, W, nc * 2) || (r > 0 && (overlaps(codes, nc, A, (uint64_t)out * r * 2) ||
                                                     overlaps(codes, nc, B, (uint64_t)r * in * 2))) ||
        overlaps(scale_out, 4, codes, nc) || overlaps(scale_out, 4, W, nc * 2))
        return LITELINEAR_ERR_INVALID_ARG;
    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return LITELINEAR_ERR_HIP;
    const bool in_capture = capturing(stream);
    litelinear_status_t st =
        grow(h->amax, (size_t)ll::residual_quant_slots(out, in) * 4, false, stream, in_capture);
    if (st != LITELINEAR_OK) return st;
    if (out == 0 || in == 0) {
        const float one = 1.0f;
        return hipMemcpyAsync(scale_out, &one, 4, hipMemcpyHostToDevice, stream) == hipSuccess &&
                       hipStreamSynchronize(stream) == hipSuccess
                   ? LITELINEAR_OK
                   : LITELINEAR_ERR_HIP;
    }
    return timed_launch(h, LITELINEAR_KERNEL_CONVERT, stream, in_capture, [&] {
        return ll::launch_residual_quant(W, r > 0 ? A : nullptr, r > 0 ? B : nullptr, out, in, r, codes,
                                         (unsigned *)h->amax.p, scale_out, stream);
    });
}

litelinear_status_t litelinear_read_probe(litelinear_handle_t h, const void *src, int64_t bytes, int work_groups,
                                         int unroll, int nontemporal, unsigned *sink, hipStream_t stream) {
    if (!h || !src || !sink || bytes <= 0 || work_groups <= 0 || work_groups > (1 << 20))
        return LITELINEAR_ERR_INVALID_ARG;
    if (bytes % 16 != 0 || !aligned(src, 16) || !aligned(sink, 4) || (unroll != 4 && unroll != 8 && unroll != 16))
        return LITELINEAR_ERR_UNSUPPORTED;
    if (overlaps(sink, (uint64_t)work_groups * 4, src, (uint64_t)bytes)) return LITELINEAR_ERR_INVALID_ARG;
    DeviceGuard guard(h->device);
    if (guard.err != hipSuccess) return LITELINEAR_ERR_HIP;
    return ll::launch_read_probe(src, bytes, work_groups, unroll, nontemporal != 0, sink, stream) == hipSuccess
               ? LITELINEAR_OK
               : LITELINEAR_ERR_HIP;
}

}  // extern "C"
