// C ABI of the fused LiteLinear forward (declared in include/litelinear.h):
// argument checks, the per-handle workspace, the choice between the skinny
// and the tiled kernels, and optional per-kernel event timing.
#include "litelinear.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <new>
#include <utility>
#include <vector>

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

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

}  // namespace

struct litelinear_ctx {
    int device = 0;
    void *t_ws = nullptr;
    size_t t_ws_bytes = 0;
    unsigned *tile_sync = nullptr;  // tiled path: counters (per row tile and per T block)
    size_t tile_sync_bytes = 0;
    float *t_part = nullptr;        // K-slice partial sums of T (both paths)
    size_t t_part_bytes = 0;
    // Launches since the counters of each path were zeroed (their T-ready
    // counters only grow, by a fixed step per launch).
    unsigned tiled_epoch = 0, skinny_epoch = 0;
    uint64_t tiled_key = 0, skinny_key = 0;  // layout the counters were last used with
    void *a_pad = nullptr;          // tiled path: zero-padded copy of A
    size_t a_pad_bytes = 0;
    void *a_pad2 = nullptr;         // ... and of a pair's second A
    size_t a_pad2_bytes = 0;
    void *t_ws2 = nullptr;          // a pair's second T' workspace
    size_t t_ws2_bytes = 0;
    float *partials = nullptr;
    size_t partials_bytes = 0;
    unsigned *counters = nullptr;
    size_t n_counters = 0;
    void *xq = nullptr;             // fp8-activation mode: e4m3fn codes of x
    size_t xq_bytes = 0;
    float *xs = nullptr;            // ... and the rows' scales
    size_t xs_bytes = 0;
    unsigned *amax = nullptr;       // decomposition side: max |R| as float bits
    size_t amax_bytes = 0;
    int64_t opt_path = 0, opt_out_f32 = 0, opt_split = 0, opt_profile = 0, opt_t_splits = 0, opt_act_fp8 = 0, opt_gelu = 0;
    Prof prof[kNumKernels];
    std::vector<hipEvent_t> event_pool;
};

namespace {

litelinear_status_t grow(void **p, size_t *have, size_t need, bool zero) {
    if (*have >= need) return LITELINEAR_OK;
    if (*p) {
        if (hipDeviceSynchronize() != hipSuccess) return LITELINEAR_ERR_HIP;
        (void)hipFree(*p);
        *p = nullptr;
        *have = 0;
    }
    if (hipMalloc(p, need) != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return LITELINEAR_ERR_OOM;
    }
    // Zeroed before any kernel of any stream can use it.
    if (zero && (hipMemset(*p, 0, need) != hipSuccess || hipDeviceSynchronize() != hipSuccess))
        return LITELINEAR_ERR_HIP;
    *have = need;
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

// Launches `fn` on `s`, bracketed by an event pair when profiling is on.
template <class F>
litelinear_status_t timed_launch(litelinear_ctx *h, int kind, hipStream_t s, F fn) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (h->opt_profile) {
        e0 = take_event(h);
        e1 = take_event(h);
        if (!e0 || !e1 || hipEventRecord(e0, s) != hipSuccess) return LITELINEAR_ERR_HIP;
    }
    if (fn() != hipSuccess) return LITELINEAR_ERR_HIP;
    if (h->opt_profile) {
        if (hipEventRecord(e1, s) != hipSuccess) return LITELINEAR_ERR_HIP;
        h->prof[kind].pending.emplace_back(e0, e1);
    }
    return LITELINEAR_OK;
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
    }
    return "unknown status";
}

namespace {

// litelinear_check_args() for x rows ldx elements apart.
litelinear_status_t check_args_ld(const void *x, int64_t ldx, const void *A, const void *B, const void *Q,
                                  const void *bias, const void *y, int64_t M, int64_t in, int64_t out, int64_t r,
                                  int y_bytes_per_elem) {
    const int64_t lim = (int64_t)1 << 40;
    if (M < 0 || in < 0 || out < 0 || r < 0) return LITELINEAR_ERR_INVALID_ARG;
    if (ldx < in || ldx > lim || (double)M * (double)ldx > 4.0e18) return LITELINEAR_ERR_INVALID_ARG;
    if (y_bytes_per_elem != 2 && y_bytes_per_elem != 4) return LITELINEAR_ERR_INVALID_ARG;
    if (M > lim || in > lim || out > lim || r > lim) return LITELINEAR_ERR_INVALID_ARG;
    if ((double)M * (double)in > 4.0e18 || (double)M * (double)out > 1.0e18 ||
        (double)out * (double)in > 4.0e18 || (double)r * (double)(in + out) > 4.0e18)
        return LITELINEAR_ERR_INVALID_ARG;
    if (M == 0 || out == 0) return LITELINEAR_OK;  // nothing to compute
    if (!y) return LITELINEAR_ERR_INVALID_ARG;
    if (in > 0 && (!x || !Q)) return LITELINEAR_ERR_INVALID_ARG;
    if (r > 0 && (!A || (in > 0 && !B))) return LITELINEAR_ERR_INVALID_ARG;
    if (in % 16 != 0) return LITELINEAR_ERR_UNSUPPORTED;
    if (in > 0 && (!aligned(x, 16) || !aligned(Q, 16) || ldx % 8 != 0)) return LITELINEAR_ERR_UNSUPPORTED;
    if (r > 0 && in > 0 && !aligned(B, 16)) return LITELINEAR_ERR_UNSUPPORTED;
    if (r > 0 && !aligned(A, 2)) return LITELINEAR_ERR_UNSUPPORTED;
    if (bias && !aligned(bias, 2)) return LITELINEAR_ERR_UNSUPPORTED;
    if (!aligned(y, (uintptr_t)y_bytes_per_elem)) return LITELINEAR_ERR_UNSUPPORTED;
    const uint64_t ny = (uint64_t)M * (uint64_t)out * (uint64_t)y_bytes_per_elem;
    // x's extent: M - 1 row strides and one row
    const uint64_t nx = in > 0 ? ((uint64_t)(M - 1) * (uint64_t)ldx + (uint64_t)in) * 2 : 0;
    if (overlaps(y, ny, x, nx) || overlaps(y, ny, Q, (uint64_t)out * in) ||
        (r > 0 && (overlaps(y, ny, A, (uint64_t)out * r * 2) || overlaps(y, ny, B, (uint64_t)r * in * 2))) ||
        overlaps(y, ny, bias, (uint64_t)out * 2))
        return LITELINEAR_ERR_INVALID_ARG;
    return LITELINEAR_OK;
}

}  // namespace

litelinear_status_t litelinear_check_args(const void *x, const void *A, const void *B, const void *Q,
                                          const void *bias, const void *y, int64_t M, int64_t in,
                                          int64_t out, int64_t r, int y_bytes_per_elem) {
    return check_args_ld(x, in, A, B, Q, bias, y, M, in, out, r, y_bytes_per_elem);
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
    *out = h;
    return LITELINEAR_OK;
}

litelinear_status_t litelinear_destroy(litelinear_handle_t h) {
    if (!h) return LITELINEAR_OK;
    litelinear_status_t st = LITELINEAR_OK;
    {
        DeviceGuard g(h->device);
        if (hipDeviceSynchronize() != hipSuccess) st = LITELINEAR_ERR_HIP;
        if (h->t_ws) (void)hipFree(h->t_ws);
        if (h->tile_sync) (void)hipFree(h->tile_sync);
        if (h->t_part) (void)hipFree(h->t_part);
        if (h->a_pad) (void)hipFree(h->a_pad);
        if (h->a_pad2) (void)hipFree(h->a_pad2);
        if (h->t_ws2) (void)hipFree(h->t_ws2);
        if (h->partials) (void)hipFree(h->partials);
        if (h->counters) (void)hipFree(h->counters);
        if (h->xq) (void)hipFree(h->xq);
        if (h->xs) (void)hipFree(h->xs);
        if (h->amax) (void)hipFree(h->amax);
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
        case LITELINEAR_OPT_ACT_FP8:
            if (value != 0 && value != 1) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_act_fp8 = value;
            return LITELINEAR_OK;
        case LITELINEAR_OPT_ACTIVATION:
            if (value != 0 && value != 1) return LITELINEAR_ERR_INVALID_ARG;
            h->opt_gelu = value;
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

}  // extern "C"

namespace {

// One output of a forward: y [M, out] = (x B^T) A^T + scale x dec(Q)^T + bias.
struct OutSet {
    const void *A, *Q, *bias;
    float scale;
    void *y;
    int64_t out;
};

// The forward for one output, or for two sharing x and B (s2 != nullptr:
// the tiled kernel, T computed once).  Arguments are already checked.
litelinear_status_t forward_impl(litelinear_ctx *h, const void *x, int64_t ldx, const void *B, const OutSet &s1,
                                 const OutSet *s2,
                                 int64_t M, int64_t in, int64_t r, hipStream_t stream) {
    const void *A = s1.A, *Q = s1.Q, *bias = s1.bias;
    void *y = s1.y;
    const float scale = s1.scale;
    const int64_t out = s1.out;
    const bool out_f32 = h->opt_out_f32 != 0;
    litelinear_status_t st = LITELINEAR_OK;

    const int64_t r_pad = r > 0 ? cdiv(r, 64) * 64 : 0;
    // The fp8-activation mode runs on the tiled kernel only (with in == 0
    // there is no residual product to run in fp8).
    const bool act8 = h->opt_act_fp8 != 0 && in > 0;
    int64_t path = h->opt_path;
    ll::SkinnyPlan plan{};
    const bool skinny_ok = !act8 && in > 0 && ll::skinny_supports(M) &&
                           ll::skinny_shape_ok(M, in, out, r_pad, plan = ll::skinny_plan(M, in, out, r_pad, h->opt_split), ldx);
    if (s2) path = 2;
    if (path == 0) path = (M <= kSkinnyAutoMaxM && skinny_ok && !ll::tiled_tiny_shape(M, in, out, r)) ? 1 : 2;
    if (path == 1 && !skinny_ok) return LITELINEAR_ERR_UNSUPPORTED;

    // A whose rows are not whole 16-byte chunks is first copied into a
    // zero-padded [out, r_pad] buffer (both paths read A in 16-byte chunks).
    const void *a_eff = A;
    if (ll::a_needs_padding(r, A)) {
        st = grow(&h->a_pad, &h->a_pad_bytes, (size_t)out * r_pad * 2, false);
        if (st != LITELINEAR_OK) return st;
        st = timed_launch(h, LITELINEAR_KERNEL_PAD_A, stream,
                          [&] { return ll::launch_pad_a(A, h->a_pad, out, r, r_pad, stream); });
        if (st != LITELINEAR_OK) return st;
        a_eff = h->a_pad;
    }
    const void *a_eff2 = s2 ? s2->A : nullptr;
    if (s2 && ll::a_needs_padding(r, s2->A)) {
        st = grow(&h->a_pad2, &h->a_pad2_bytes, (size_t)s2->out * r_pad * 2, false);
        if (st != LITELINEAR_OK) return st;
        st = timed_launch(h, LITELINEAR_KERNEL_PAD_A, stream,
                          [&] { return ll::launch_pad_a(s2->A, h->a_pad2, s2->out, r, r_pad, stream); });
        if (st != LITELINEAR_OK) return st;
        a_eff2 = h->a_pad2;
    }

    if (path == 1) {
        ll::SkinnyProblem p{};
        p.plan = plan;
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
        p.gelu = h->opt_gelu != 0;
        if (p.plan.splits > 1) {
            st = grow((void **)&h->partials, &h->partials_bytes, (size_t)p.plan.splits * M * out * sizeof(float),
                      false);
            if (st != LITELINEAR_OK) return st;
            p.partials = h->partials;
        }
        if (r > 0) {
            st = grow((void **)&h->t_part, &h->t_part_bytes, (size_t)p.plan.t_splits * M * r_pad * sizeof(float),
                      false);
            if (st != LITELINEAR_OK) return st;
            p.t_part = h->t_part;
        }
        size_t cbytes = h->n_counters * sizeof(unsigned);
        const size_t need = (size_t)ll::skinny_sync_words(p.plan) * sizeof(unsigned);
        if (cbytes < need) h->skinny_epoch = 0;  // counters start again from zero
        st = grow((void **)&h->counters, &cbytes, need, true);
        if (st != LITELINEAR_OK) return st;
        h->n_counters = cbytes / sizeof(unsigned);
        p.sync = h->counters;
        // The T flag sits after the column-tile counters: a new layout or
        // step (with or without T) starts every counter again from zero, so
        // no word ever holds another layout's flag.
        const uint64_t key = ((uint64_t)p.plan.tiles_n << 32) | (uint64_t)(r > 0 ? p.plan.pps * p.plan.splits : 0);
        if (key != h->skinny_key) {
            if (hipMemsetAsync(h->counters, 0, cbytes, stream) != hipSuccess) return LITELINEAR_ERR_HIP;
            h->skinny_key = key;
            h->skinny_epoch = 0;
        }
        p.t_target = (h->skinny_epoch + 1u) * (unsigned)(p.plan.pps * p.plan.splits);
        st = timed_launch(h, LITELINEAR_KERNEL_SKINNY, stream, [&] { return ll::launch_skinny(p, a_eff, stream); });
        if (st == LITELINEAR_OK && r > 0) ++h->skinny_epoch;
        return st;
    }

    ll::TiledProblem p{};
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
    p.gelu = h->opt_gelu != 0;
    if (s2) {
        p.Q2 = s2->Q;
        p.A2 = s2->A;
        p.bias2 = s2->bias;
        p.y2 = s2->y;
        p.scale2 = s2->scale;
        p.N2 = s2->out;
    }
    const ll::TileCfg mc = ll::choose_main_tile(p);
    if (!ll::tiled_shape_ok(p, mc)) return LITELINEAR_ERR_UNSUPPORTED;
    if (act8) {
        st = grow(&h->xq, &h->xq_bytes, (size_t)M * in, false);
        if (st != LITELINEAR_OK) return st;
        st = grow((void **)&h->xs, &h->xs_bytes, (size_t)M * sizeof(float), false);
        if (st != LITELINEAR_OK) return st;
        st = timed_launch(h, LITELINEAR_KERNEL_QUANT, stream,
                          [&] { return ll::launch_quant_rows(x, ldx, h->xq, h->xs, M, in, stream); });
        if (st != LITELINEAR_OK) return st;
        p.xq = h->xq;
        p.xs = h->xs;
    }
    // With producers, T goes through the T' workspace and the row tiles'
    // ready counters; small problems compute it in each output tile instead.
    const bool producers = r > 0 && !ll::tiled_self_t(p, mc);
    if (producers) {
        st = grow(&h->t_ws, &h->t_ws_bytes, (size_t)M * r_pad * 2, false);
        if (st != LITELINEAR_OK) return st;
        p.t_ws = h->t_ws;
        if (s2) {
            st = grow(&h->t_ws2, &h->t_ws2_bytes, (size_t)M * r_pad * 2, false);
            if (st != LITELINEAR_OK) return st;
            p.t_ws2 = h->t_ws2;
        }
        p.t_splits = ll::tiled_t_splits(p, mc, h->opt_t_splits);
        if (p.t_splits > 1) {
            st = grow((void **)&h->t_part, &h->t_part_bytes, (size_t)p.t_splits * M * r_pad * sizeof(float), false);
            if (st != LITELINEAR_OK) return st;
            p.t_part = h->t_part;
        }
        const size_t need = (size_t)ll::tiled_sync_words(p, mc) * sizeof(unsigned);
        if (h->tile_sync_bytes < need) h->tiled_epoch = 0;  // counters start again from zero
        st = grow((void **)&h->tile_sync, &h->tile_sync_bytes, need, true);
        if (st != LITELINEAR_OK) return st;
        // The ready counters of every row tile must have grown by the same
        // step in every launch so far; a different row-tile count or step
        // starts them again from zero (ordered on the stream).
        const uint64_t key = ((uint64_t)ll::tiled_row_tiles(p, mc) << 32) | ll::tiled_flag_step(p, mc);
        if (key != h->tiled_key) {
            if (hipMemsetAsync(h->tile_sync, 0, h->tile_sync_bytes, stream) != hipSuccess) return LITELINEAR_ERR_HIP;
            h->tiled_key = key;
            h->tiled_epoch = 0;
        }
        p.t_target = (h->tiled_epoch + 1u) * ll::tiled_flag_step(p, mc);
    }
    st = timed_launch(h, LITELINEAR_KERNEL_MAIN, stream,
                      [&] { return ll::launch_tiled(p, mc, a_eff, a_eff2, h->tile_sync, stream); });
    if (st == LITELINEAR_OK && producers) ++h->tiled_epoch;
    return st;
}

}  // namespace

extern "C" {

litelinear_status_t litelinear_forward_strided(litelinear_handle_t h, const void *x, int64_t ldx, const void *A,
                                               const void *B, const void *Q, float scale, const void *bias, void *y,
                                               int64_t M, int64_t in, int64_t out, int64_t r, hipStream_t stream) {
    if (!h) return LITELINEAR_ERR_INVALID_ARG;
    const bool out_f32 = h->opt_out_f32 != 0;
    litelinear_status_t st = check_args_ld(x, ldx, A, B, Q, bias, y, M, in, out, r, out_f32 ? 4 : 2);
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

litelinear_status_t litelinear_forward_pair(litelinear_handle_t h, const void *x, const void *B, const void *A1,
                                            const void *Q1, float scale1, const void *bias1, void *y1, int64_t out1,
                                            const void *A2, const void *Q2, float scale2, const void *bias2, void *y2,
                                            int64_t out2, int64_t M, int64_t in, int64_t r, hipStream_t stream) {
    if (!h) return LITELINEAR_ERR_INVALID_ARG;
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
    const bool skinny = h->opt_path == 1 || (h->opt_path == 0 && M <= kSkinnyAutoMaxM && h->opt_act_fp8 == 0);
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
    return timed_launch(h, LITELINEAR_KERNEL_QUANT, stream,
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
    litelinear_status_t st = grow((void **)&h->amax, &h->amax_bytes, 256, false);
    if (st != LITELINEAR_OK) return st;
    if (n == 0) {
        const float one = 1.0f;  // scale of an empty (all-zero) tensor
        return hipMemcpyAsync(scale_out, &one, 4, hipMemcpyHostToDevice, stream) == hipSuccess &&
                       hipStreamSynchronize(stream) == hipSuccess
                   ? LITELINEAR_OK
                   : LITELINEAR_ERR_HIP;
    }
    return timed_launch(h, LITELINEAR_KERNEL_CONVERT, stream,
                        [&] { return ll::launch_quant_tensor(R, n, codes, h->amax, scale_out, stream); });
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
    litelinear_status_t st = grow((void **)&h->amax, &h->amax_bytes, 256, false);
    if (st != LITELINEAR_OK) return st;
    if (out == 0 || in == 0) {
        const float one = 1.0f;
        return hipMemcpyAsync(scale_out, &one, 4, hipMemcpyHostToDevice, stream) == hipSuccess &&
                       hipStreamSynchronize(stream) == hipSuccess
                   ? LITELINEAR_OK
                   : LITELINEAR_ERR_HIP;
    }
    return timed_launch(h, LITELINEAR_KERNEL_CONVERT, stream, [&] {
        return ll::launch_residual_quant(W, r > 0 ? A : nullptr, r > 0 ? B : nullptr, out, in, r, codes, h->amax,
                                         scale_out, stream);
    });
}

}  // extern "C"
