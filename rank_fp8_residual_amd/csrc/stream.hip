// Stream path of the fused LiteLinear forward on gfx950: one row block
// (M <= 16) against a wide output, HBM-bound on reading Q once.
//
// The forward (LiteLinear README, page "moonmath-ai/LiteLinear", equation in
// the introduction):  y = (x B^T) A^T + scale * (x dec(Q)^T) + bias.
//
// One launch of two kinds of work-group:
//   * T producers (the lowest ids): 16 per group of 64 ranks, each computing
//     T = x B^T for its 64 ranks over one sixteenth of K (all loads of the
//     piece in flight at once), stored as float32; the last of a group's
//     sixteen to finish (a counter) adds the pieces in K order, rounds T once
//     to bf16 and announces the group.  They run at the start, beside the
//     streams, and are done long before anyone needs T.
//   * Streamers: one per 32 output columns, over all of K, so that no
//     partial sums cross work-groups.  Each wave streams a quarter of K:
//     per 64-element step, 16 rows x 64 codes of each of its two column
//     fragments (non-temporal 16-byte loads, every load instruction whole
//     64-byte lines) and the matching 16 x 64 bf16 of x (from L2: x is
//     small and every streamer reads all of it once), DEPTH steps in flight,
//     codes converted exactly to bf16 right before v_mfma_f32_16x16x32_bf16.
//     Wave 0 then adds the four quarters in wave order (through LDS), forms
//     scale * sum + T A^T + bias (T and A requested before the stream's end)
//     and stores y.
// The work-groups of one launch fit on the device together (a streamer
// takes 4 waves and at most 128 VGPRs each), producers are dispatched
// first and wait for nothing, and streamers wait for T only after their
// streams; the wait is bounded and a wait that gives up sets the error
// word.  The counters are back at zero when the launch ends: each group's
// piece counter is cleared by its summer, the T-ready counter by the last
// streamer to have read T.
#include "device_common.hpp"
#include "launch.hpp"

namespace ll {
namespace {

constexpr int XNT = 256;       // threads per work-group
constexpr int XCOLS = 32;      // products' columns per streamer (two fragments)
constexpr int TK_SPLIT = 16;   // producers per group of 64 ranks (K sixteenths)
constexpr int TPIECE = 16 * 64;  // floats per piece (16 rows x 64 ranks)

struct XArgs {
    const unsigned char *x, *B, *Q, *A, *bias;
    void *y;
    unsigned char *t;      // T bf16 [16, r_pad]
    float *tpiece;         // pieces float32 [groups][TK_SPLIT][16][64]
    unsigned *pcnt;        // per rank group: pieces finished
    unsigned *tready;      // rank groups finished
    unsigned *done;        // streamers done reading T
    unsigned *err;
    unsigned wait_limit, t_target;
    float scale;
    int M, K, N, r, r_pad, lda, ldx;
    int producers, groups, kpiece;   // producer work-groups, rank groups, K per piece (multiple of 32)
    int streamers;
    int steps;             // 64-element K steps of one wave's quarter
    bool y_vec, out_f32, gelu;
    bool glu;              // gated epilogue (see skinny.hip): fragment 0 hidden, 1 gate
    int F, NO;             // gate half, output columns
};

// ---------------------------------------------------------------- producers

__device__ __forceinline__ void t_producer(const XArgs &a, int pid, unsigned char *lds) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
    const int grp = pid / TK_SPLIT, kr = pid - grp * TK_SPLIT;
    const int k0 = kr * a.kpiece;
    // wave w: ranks 64 grp + 16 w .. +16 over K [k0, k0 + kpiece)
    const int rank0 = 64 * grp + 16 * wave;
    const rsrc_t rb = make_rsrc(a.B, (int64_t)a.r * a.K * 2);
    const rsrc_t rx = make_rsrc(a.x, (int64_t)a.M * a.ldx * 2);
    // chunks of 32 K, CB per round of loads (all of a round in flight)
    constexpr int CB = 8;
    const int kend = k0 + a.kpiece < a.K ? k0 + a.kpiece : a.K;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int cb = 0; cb < a.kpiece / 32; cb += CB) {
        u32x4 bv[CB], xv[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int k = k0 + 32 * (cb + c) + 8 * g;
            const bool ok = k < kend;
            bv[c] = bload16(rb, ((unsigned)(rank0 + l16) * (unsigned)a.K + (unsigned)k) * 2u +
                                    (ok && rank0 + l16 < a.r ? 0u : kOOB));
            xv[c] = bload16(rx, ((unsigned)l16 * (unsigned)a.ldx + (unsigned)k) * 2u + (ok ? 0u : kOOB));
        }
#pragma unroll
        for (int c = 0; c < CB; ++c) acc = mfma16(bv[c], xv[c], acc);
    }
    // lane holds T[m = l16][rank rank0 + 4 g + v] partial over the piece's K
    float *piece = a.tpiece + ((int64_t)grp * TK_SPLIT + kr) * TPIECE;
    const rsrc_t rp = make_rsrc(piece, TPIECE * 4);
    bstore16<kDeviceCoherent>(rp, (unsigned)((l16 * 64 + 16 * wave + 4 * g) * 4), __builtin_bit_cast(u32x4, acc));
    unsigned *is_last = reinterpret_cast<unsigned *>(lds);
    wait_vmcnt<0>();
    __syncthreads();
    if (tid == 0) *is_last = bump_u32(&a.pcnt[grp]) == (unsigned)(TK_SPLIT - 1) ? 1u : 0u;
    __syncthreads();
    if (!*is_last) return;
    // Sum of the group's pieces in K order: thread t owns elements 4t .. 4t+3
    // of the 16 x 64 block (row t / 16, ranks 4 (t % 16) ..).
    const rsrc_t rall = make_rsrc(a.tpiece + (int64_t)grp * TK_SPLIT * TPIECE, TK_SPLIT * TPIECE * 4);
    f32x4 p[TK_SPLIT];
#pragma unroll
    for (int q = 0; q < TK_SPLIT; ++q) p[q] = bload16f_dc(rall, (unsigned)((q * TPIECE + 4 * tid) * 4));
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < TK_SPLIT; ++q) s += p[q];
    const int row = tid >> 4, col = 64 * grp + 4 * (tid & 15);
    const rsrc_t rt = make_rsrc(a.t, (int64_t)16 * a.r_pad * 2);
    bstore8<kDeviceCoherent>(rt, (unsigned)((row * a.r_pad + col) * 2),
                             u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])});
    wait_vmcnt<0>();
    __syncthreads();
    if (tid == 0) {
        __hip_atomic_store(&a.pcnt[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bump_u32(a.tready);
    }
}

// ---------------------------------------------------------------- streamers

template <int QF, int D>
__device__ __forceinline__ void streamer(const XArgs &a, int sid, unsigned char *lds) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
    const int n0 = sid * XCOLS;
    // Q / A row of this lane in fragment f (relative to the tensors' starts),
    // or past the end when it does not exist.
    const int c0 = sid * (XCOLS / 2);  // gated epilogue: first output column
    auto wrow = [&](int f) -> unsigned {
        if (a.glu) return c0 + l16 < a.F ? (unsigned)(f * a.F + c0 + l16) : 0x7FFFFFFFu;
        return n0 + 16 * f + l16 < a.N ? (unsigned)(n0 + 16 * f + l16) : 0x7FFFFFFFu;
    };
    const int nrows = a.glu ? 2 * a.F : a.N;
    const rsrc_t rq = make_rsrc(a.Q, (int64_t)nrows * a.K);
    const rsrc_t rx = make_rsrc(a.x, (int64_t)a.M * a.ldx * 2);
    // (a missing row's offset has the out-of-range bit set; the K offset is
    // OR-ed in, so no sum wraps back into range)
    unsigned qoff[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const unsigned row = wrow(f);
        qoff[f] = row == 0x7FFFFFFFu ? kOOB : row * (unsigned)a.K;
    }
    const unsigned xoff = (unsigned)l16 * (unsigned)a.ldx * 2u;
    // this wave's quarter of the K steps
    const int s0 = wave * a.steps;
    const int kend = (s0 + a.steps) * 64 < a.K ? (s0 + a.steps) * 64 : a.K;

    // Bias and the first 64 ranks of A, requested up front.
    const rsrc_t rb = make_rsrc(a.bias, a.bias ? (int64_t)nrows * 2 : 0);
    const rsrc_t ra = make_rsrc(a.A, (int64_t)nrows * a.lda * 2);
    float bv[2][4];
    u32x4 af[2][2];
    if (wave == 0) {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int cc = a.glu ? c0 + 4 * g + v : n0 + 16 * f + 4 * g + v;
                const int idx = a.glu ? f * a.F + cc : cc;
                const bool ok = a.glu ? cc < a.F : cc < a.N;
                bv[f][v] = bload_bf16(rb, (unsigned)idx + (ok ? 0u : kOOB / 2));
            }
            const unsigned row = wrow(f);
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int ka = 32 * c + 8 * g;
                af[f][c] = bload16(ra, ka < a.lda && row != 0x7FFFFFFFu && a.r > 0
                                           ? (row * (unsigned)a.lda + (unsigned)ka) * 2u
                                           : kOOB);
            }
        }
    }

    // Lane holds codes [k + 16 g, +16) of its fragment rows and x[l16][k + 16 g, +16).
    u32x4 qr[D][2], xr[D][2];
    auto load = [&](int slot, int s) {
        const int k = (s0 + s) * 64 + 16 * g;
        const unsigned oob = k < kend ? 0u : kOOB;
#pragma unroll
        for (int f = 0; f < 2; ++f)
            qr[slot][f] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, ((qoff[f] + (unsigned)k) | oob), 0, 2 /* nt */));
        const unsigned xo = xoff + (unsigned)k * 2u + oob;
        xr[slot][0] = bload16(rx, xo);
        xr[slot][1] = bload16(rx, xo + 16u);
    };
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < D - 1; ++s) load(s, s);
    // The loop runs in blocks of D steps (ring slots indexed statically);
    // steps past the wave's quarter load zeros and add nothing.
    const int blocks = (a.steps + D - 1) / D;
    for (int bk = 0; bk < blocks; ++bk) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int s = bk * D + u;
            load((u + D - 1) % D, s + D - 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const u32x4 q = qr[u][f];
                u32x4 h0, h1;
                if constexpr (QF == 0) {
                    fp8x16_to_bf16x16(q, h0, h1);
                } else {
                    u32x2 c[4] = {q8x4_to_bf16x4<1>(q.x), q8x4_to_bf16x4<1>(q.y), q8x4_to_bf16x4<1>(q.z),
                                  q8x4_to_bf16x4<1>(q.w)};
                    const unsigned sp =
                        fnuz_special_or(fnuz_special_or(fnuz_special_or(fnuz_special_or(0u, q.x), q.y), q.z), q.w);
                    if (fnuz_any_special(sp)) {
                        c[0] = fnuz_patch(q.x, c[0]);
                        c[1] = fnuz_patch(q.y, c[1]);
                        c[2] = fnuz_patch(q.z, c[2]);
                        c[3] = fnuz_patch(q.w, c[3]);
                    }
                    h0 = u32x4{c[0].x, c[0].y, c[1].x, c[1].y};
                    h1 = u32x4{c[2].x, c[2].y, c[3].x, c[3].y};
                }
                acc[f] = mfma16(h0, xr[u][0], acc[f]);
                acc[f] = mfma16(h1, xr[u][1], acc[f]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    wait_vmcnt<0>();  // the ring's last (zero) loads

    // The quarters in wave order: waves 1..3 leave theirs in LDS.
    f32x4 *red = reinterpret_cast<f32x4 *>(lds);
    if (wave > 0) {
        red[((wave - 1) * 2 + 0) * 64 + lane] = acc[0];
        red[((wave - 1) * 2 + 1) * 64 + lane] = acc[1];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        acc[0] += red[(w * 2 + 0) * 64 + lane];
        acc[1] += red[(w * 2 + 1) * 64 + lane];
    }
    acc[0] *= a.scale;
    acc[1] *= a.scale;

    if (a.r > 0) {
        // T: announced by the producers long ago (bounded wait, reported).
        unsigned spins = 0;
        while (__builtin_amdgcn_readfirstlane(poll_u32(a.tready)) < a.t_target) {
            if (++spins >= a.wait_limit) {
                if (lane == 0) report_wait_timeout(a.err);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        const rsrc_t rt = make_rsrc(a.t, (int64_t)16 * a.r_pad * 2);
        for (int h = 0; h < a.r_pad / 64; ++h) {
            u32x4 afh[2][2];
            if (h == 0) {
#pragma unroll
                for (int f = 0; f < 2; ++f)
#pragma unroll
                    for (int c = 0; c < 2; ++c) afh[f][c] = af[f][c];
            } else {
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    const unsigned row = wrow(f);
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const int ka = 64 * h + 32 * c + 8 * g;
                        afh[f][c] = bload16(ra, ka < a.lda && row != 0x7FFFFFFFu
                                                    ? (row * (unsigned)a.lda + (unsigned)ka) * 2u
                                                    : kOOB);
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                // lane: T[l16][64 h + 32 c + 8 g, +8), device-coherent
                const u32x4 tf = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               rt, (unsigned)((l16 * a.r_pad + 64 * h + 32 * c + 8 * g) * 2), 0, kDeviceCoherent));
#pragma unroll
                for (int f = 0; f < 2; ++f) acc[f] = mfma16(afh[f][c], tf, acc[f]);
            }
        }
        // every T read of this wave has landed (the products used them); the
        // launch's last streamer clears the T counters
        if (lane == 0 && bump_u32(a.done) == (unsigned)(a.streamers - 1)) {
            __hip_atomic_store(a.tready, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // y: lane holds row m = l16, columns 4 g .. 4 g + 3 of fragment f
    const int m = l16;
    auto emit = [&](int n, const float (&o0)[4]) {
        if (m >= a.M || n >= a.NO) return;
        float o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = a.gelu ? gelu_tanh(o0[v]) : o0[v];
        if (a.out_f32) {
            float *dst = reinterpret_cast<float *>(a.y) + (int64_t)m * a.NO + n;
            if (a.y_vec && n + 3 < a.NO) {
                *reinterpret_cast<f32x4 *>(dst) = f32x4{o[0], o[1], o[2], o[3]};
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (n + v < a.NO) dst[v] = o[v];
            }
        } else {
            unsigned short *dst = reinterpret_cast<unsigned short *>(a.y) + (int64_t)m * a.NO + n;
            if (a.y_vec && n + 3 < a.NO) {
                *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (n + v < a.NO) dst[v] = f32_to_bf16_rne(o[v]);
            }
        }
    };
    if (a.glu) {
        float o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = (acc[0][v] + bv[0][v]) * gelu_erf(acc[1][v] + bv[1][v]);
        emit(c0 + 4 * g, o);
    } else {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const float o[4] = {acc[f][0] + bv[f][0], acc[f][1] + bv[f][1], acc[f][2] + bv[f][2],
                                acc[f][3] + bv[f][3]};
            emit(n0 + 16 * f + 4 * g, o);
        }
    }
}

template <int QF, int D>
__global__ void __launch_bounds__(XNT) stream_kernel(XArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[6 * 64 * 16];
    const int b = (int)blockIdx.x;
    if (b < a.producers) {
        t_producer(a, b, lds);
        return;
    }
    streamer<QF, D>(a, b - a.producers, lds);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace
}  // namespace ll

// ------------------------------------------------------------------ host

namespace ll {

namespace {
constexpr int kStreamMinWGs = 128;  // below this many column tiles the split-K kernel fills the chip better
}

bool stream_supports(int64_t M, int64_t K, int64_t N, int64_t r_pad, bool glu, int64_t ldx) {
    const int64_t lim = (int64_t)1 << 31;
    const int64_t cols = glu ? N / 2 : N;            // output columns
    const int64_t wgs = glu ? cdiv(cols, XCOLS / 2) : cdiv(N, XCOLS);
    const int64_t groups = r_pad / 64;
    return M >= 1 && M <= 16 && K > 0 && wgs >= kStreamMinWGs && N * K < lim && N * (r_pad > 0 ? r_pad : 1) * 2 < lim &&
           (int64_t)r_pad * K * 2 < lim && 16 * ldx * 2 < lim && wgs + TK_SPLIT * groups < lim &&
           TK_SPLIT * groups <= 256 && K < lim / 2;
}

int64_t stream_sync_words(int64_t r_pad) { return r_pad / 64 + 2; }
int64_t stream_piece_bytes(int64_t r_pad) { return (r_pad / 64) * TK_SPLIT * TPIECE * 4; }
int64_t stream_t_bytes(int64_t r_pad) { return 16 * r_pad * 2; }

hipError_t launch_stream(const StreamProblem &p, const void *a_eff, hipStream_t s) {
    XArgs a{};
    a.x = (const unsigned char *)p.x;
    a.ldx = (int)p.ldx;
    a.B = (const unsigned char *)p.B;
    a.Q = (const unsigned char *)p.Q;
    a.A = (const unsigned char *)a_eff;
    a.bias = (const unsigned char *)p.bias;
    a.y = p.y;
    a.scale = p.scale;
    a.M = (int)p.M;
    a.K = (int)p.K;
    a.N = (int)p.N;
    a.r = (int)p.r;
    a.r_pad = (int)p.r_pad;
    a.lda = a_eff == p.A ? (int)p.r : (int)p.r_pad;
    if (p.glu && p.N % 2 != 0) return hipErrorInvalidValue;
    a.glu = p.glu;
    a.F = p.glu ? (int)(p.N / 2) : 0;
    a.NO = p.glu ? a.F : (int)p.N;
    a.streamers = p.glu ? (int)cdiv(a.F, XCOLS / 2) : (int)cdiv(p.N, XCOLS);
    a.groups = (int)(p.r_pad / 64);
    a.producers = p.r > 0 ? TK_SPLIT * a.groups : 0;
    a.kpiece = (int)(cdiv(cdiv(p.K, TK_SPLIT), 32) * 32);
    a.steps = (int)cdiv(cdiv(p.K, 64), 4);
    a.t = (unsigned char *)p.t;
    a.tpiece = p.t_piece;
    if (p.r > 0) {
        if (!p.sync || !p.t || !p.t_piece || !p.err || p.wait_limit == 0) return hipErrorInvalidValue;
        a.pcnt = p.sync;
        a.tready = p.sync + a.groups;
        a.done = p.sync + a.groups + 1;
    }
    a.err = p.err;
    a.wait_limit = p.wait_limit;
    a.t_target = (unsigned)a.groups + p.wait_extra;
    a.y_vec = (a.NO % 4 == 0) && ((uintptr_t)p.y % 16 == 0);
    a.out_f32 = p.out_f32;
    a.gelu = p.gelu;
    const int grid = a.producers + a.streamers;
    if (p.q_format)
        hipLaunchKernelGGL((stream_kernel<1, 8>), dim3(grid), dim3(XNT), 0, s, a);
    else
        hipLaunchKernelGGL((stream_kernel<0, 8>), dim3(grid), dim3(XNT), 0, s, a);
    return hipGetLastError();
}

}  // namespace ll
