// Skinny-M (HBM-bound) path of the fused LiteLinear forward on gfx950.
//
// The forward (LiteLinear README, page "moonmath-ai/LiteLinear", equation in
// the introduction):  y = (x B^T) A^T + scale * (x dec(Q)^T) + bias.
//
// With few rows the time is the time to stream Q (out * in bytes) from HBM
// once, so the launch is organised around that stream:
//   * Work-groups own 128 output columns over one K slice.  Each copies its
//     slice of x into LDS once (buffer loads straight to LDS), then its four
//     waves stream their 32 columns of Q codes with 128-bit loads into
//     registers, DEPTH steps of 64 ahead, convert them exactly to bf16 and
//     feed v_mfma_f32_16x16x32_bf16 against the x rows read from LDS.
//   * When r > 0 the lowest-id work-groups of each slice also compute pieces
//     of T = x B^T (16 ranks over part of their slice, x from the same LDS)
//     before their Q stream starts: float32, summed over the four waves in
//     wave order, stored with device-coherent stores; each piece bumps a flag.
//   * With several K slices each output work-group writes its partial sum
//     (float32, device-coherent stores); the last one of a column tile to
//     finish (an atomic counter) adds the slices in slice order, so the
//     result does not depend on which one finishes last.
//   * That last work-group then waits for T (long since done), adds the
//     pieces of T in K order, rounds T once to bf16, forms
//     scale * sum + T A^T + bias and stores y.  The slice counters are left
//     at zero; the T flag only grows, by the producer count per launch, and
//     each launch waits for its own target value.
// Only final work-groups wait, and only for T pieces.  The piece work-groups
// have the lowest ids (at most one per CU), so they are dispatched first and
// compute their pieces before waiting for anything: the waits always end.
// Every global load is a buffer load: reads past a descriptor's end return
// zero, so masking rows, columns and the K tail needs no branch.
#include "device_common.hpp"
#include "launch.hpp"

namespace ll {
namespace {

constexpr int SNT = 256;           // threads per work-group (4 waves)
constexpr int WNF = 2;             // 16-column fragments per wave
constexpr int SBN = 4 * WNF * 16;  // output columns per work-group
constexpr int SMAX_M = 64;         // largest M (4 row blocks of 16)
constexpr int DEPTH = 8;           // K steps of Q in flight per wave
constexpr int TCH = 256;           // K elements per producer load round
constexpr int XPAD = 8;            // bf16 of padding per LDS row of x
constexpr int LDS_MAX = 160 * 1024;

struct SArgs {
    const unsigned char *x, *B, *Q, *A, *bias;
    void *y;
    float *partials;     // [splits, M, N]
    unsigned *cnt;       // [tiles_n] K slices done per column tile
    unsigned *tflag;     // T pieces finished, counted over all launches
    unsigned t_target;   // tflag value meaning "this launch's T is complete" (mod 2^32)
    float *tpart;        // T pieces, float32 [t_splits, r_pad / 16, M, 16]
    float scale;
    int M, K, N, r, r_pad, lda, splits, tiles_n, t_splits;
    int ldx;             // elements between rows of x (>= K)
    int pps;             // T pieces per K slice (16 ranks x a part of the slice each)
    int pwg;             // work-groups of a slice that compute pieces (lowest ids)
    bool y_vec, out_f32, gelu;
};

// ------------------------------------------------------------ output tiles

__device__ __forceinline__ void store_out(const SArgs &a, int m, int n, const float (&y)[4]) {
    float o[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) o[v] = a.gelu ? gelu_tanh(y[v]) : y[v];
    if (a.out_f32) {
        float *dst = reinterpret_cast<float *>(a.y) + (int64_t)m * a.N + n;
        if (a.y_vec && n + 3 < a.N) {
            *reinterpret_cast<f32x4 *>(dst) = f32x4{o[0], o[1], o[2], o[3]};
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (n + v < a.N) dst[v] = o[v];
        }
    } else {
        unsigned short *dst = reinterpret_cast<unsigned short *>(a.y) + (int64_t)m * a.N + n;
        if (a.y_vec && n + 3 < a.N) {
            *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (n + v < a.N) dst[v] = f32_to_bf16_rne(o[v]);
        }
    }
}

template <int MB, int NSTEPS>
constexpr int x_lds_bytes() {
    return MB * 16 * (NSTEPS * 64 + XPAD) * 2;
}

// K elements of a T piece handled by one wave (a piece spans 4 of these).
template <int NSTEPS>
constexpr int t_kwave() {
    return NSTEPS * 16 < 256 ? NSTEPS * 16 : 256;
}

template <int MB, int NSTEPS>
__global__ void __launch_bounds__(SNT) skinny_kernel(SArgs a) {
    constexpr int KS = NSTEPS * 64;            // K elements per slice
    constexpr int XS = (KS + XPAD) * 2;        // LDS bytes per row of x
    constexpr int D = DEPTH < NSTEPS ? DEPTH : NSTEPS;
    constexpr int KW = t_kwave<NSTEPS>();      // K of a T piece per wave
    constexpr int KP = 4 * KW;                 // K of a T piece
    __shared__ __attribute__((aligned(16))) unsigned char xs[x_lds_bytes<MB, NSTEPS>()];
    __shared__ f32x4 red[4 * MB * 64];
    __shared__ unsigned is_last, tflag_sh;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
    // Work-group id -> (slice, column tile): the pwg piece work-groups of
    // every slice come first.
    const int c = (int)blockIdx.x;
    int slice, tn;
    const bool piece_wg = c < a.pwg * a.splits;
    if (piece_wg) {
        slice = c / a.pwg;
        tn = c - slice * a.pwg;
    } else {
        const int c2 = c - a.pwg * a.splits, rest = a.tiles_n - a.pwg;
        slice = c2 / rest;
        tn = a.pwg + (c2 - slice * rest);
    }
    const int n0 = tn * SBN, nw = n0 + wave * (WNF * 16);
    const int kb = slice * KS;
    const int rows_n = (a.N - n0) < SBN ? (a.N - n0) : SBN;

    // Uniform descriptors (built here so they stay in scalar registers).
    const rsrc_t rq = make_rsrc(a.Q + (int64_t)n0 * a.K, (int64_t)rows_n * a.K);
    const rsrc_t rx = make_rsrc(a.x, (int64_t)a.M * a.ldx * 2);
    const rsrc_t rp = make_rsrc(a.partials, a.splits > 1 ? (int64_t)a.splits * a.M * a.N * 4 : 0);
    const rsrc_t rb = make_rsrc(a.bias, a.bias ? (int64_t)a.N * 2 : 0);

    // Bias of this lane's columns, requested first (past N and a missing
    // bias read as zero).
    float bv[WNF][4];
#pragma unroll
    for (int f = 0; f < WNF; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v) bv[f][v] = bload_bf16(rb, (unsigned)(nw + 16 * f + 4 * g + v));

    // The first 64 ranks of this lane's A rows, also requested up front: A is
    // read from HBM for the first time, and only a final work-group (any
    // work-group may be one) uses it, after its Q stream.
    const rsrc_t ra = make_rsrc(a.A + (int64_t)n0 * a.lda * 2, (int64_t)rows_n * a.lda * 2);
    auto load_a = [&](u32x4 (&af)[2][WNF], int h) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int f = 0; f < WNF; ++f) {
                const int ka = 64 * h + 32 * c + 8 * g;
                af[c][f] = bload16(ra, ((unsigned)(wave * (WNF * 16) + 16 * f + l16) * (unsigned)a.lda + (unsigned)ka) *
                                               2u +
                                           (ka < a.lda ? 0u : kOOB));
            }
    };
    u32x4 af0[2][WNF];
    if (a.r > 0) load_a(af0, 0);

    // x[:, kb : kb + KS] -> LDS, rows of XS bytes (the padding puts the 16
    // rows a fragment read touches on distinct banks).  One instruction
    // moves 1 KB (512 elements) of one row; instruction i goes to wave i % 4.
    {
        constexpr int PER_ROW = KS / 512;
        const int total = a.M * PER_ROW;
        for (int i = wave; i < total; i += 4) {
            const int row = i / PER_ROW, j = i - row * PER_ROW;
            const int k = kb + 512 * j + 8 * lane;
            const unsigned off = ((unsigned)row * (unsigned)a.ldx + (unsigned)k) * 2u + (k < a.K ? 0u : kOOB);
            bload16_lds(rx, xs + row * XS + 1024 * j, off);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // T pieces: piece p of this slice is 16 ranks (fragment p % nfrag) over
    // elements [KP (p / nfrag), +KP) of the slice; wave w takes quarter w.
    // Lane holds B[16 f + l16][k + 8 g, +8) for its k steps of 32.
    const int nfrag = a.r_pad / 16;
    const rsrc_t rbm = make_rsrc(a.B, (int64_t)a.r * a.K * 2);
    auto load_b = [&](u32x4 (&bb)[KW / 32], int p) {
        const int f = p % nfrag, q = p / nfrag;
#pragma unroll
        for (int s2 = 0; s2 < KW / 32; ++s2) {
            const int k = kb + q * KP + wave * KW + 32 * s2 + 8 * g;
            bb[s2] = bload16(rbm, ((unsigned)(16 * f + l16) * (unsigned)a.K + (unsigned)k) * 2u + (k < a.K ? 0u : kOOB));
        }
    };
    u32x4 bfirst[KW / 32];
    const bool has_piece = piece_wg && a.r > 0;
    if (has_piece) load_b(bfirst, tn);

    // Q: lane holds codes [k + 16 g, +16) of row nw + 16 f + l16.
    auto load_q = [&](u32x4 (&q)[WNF], int s) {
        const int k = kb + 64 * s + 16 * g;
        const unsigned oob = k < a.K ? 0u : kOOB;
#pragma unroll
        for (int f = 0; f < WNF; ++f)
            q[f] = bload16(rq, (unsigned)(wave * (WNF * 16) + 16 * f + l16) * (unsigned)a.K + (unsigned)k + oob);
    };
    u32x4 qr[D][WNF];
#pragma unroll
    for (int s = 0; s < D - 1; ++s) load_q(qr[s], s);
    // This wave's x copies (and B loads) are older than the D - 1 steps of
    // Q loads just issued: once at most that many are in flight they have
    // landed; the barrier then covers every wave's.
    wait_vmcnt<(D - 1) * WNF>();
    __syncthreads();

    // This work-group's T pieces: 16 ranks x KW per wave from LDS x, the
    // four quarters added in wave order through LDS by wave 0, stored
    // device-coherent as float32 piece [slice (KS / KP) + p / nfrag][f][m][16].
    if (has_piece) {
        const rsrc_t rtp = make_rsrc(a.tpart, (int64_t)a.t_splits * nfrag * a.M * 16 * 4);
        auto piece = [&](const u32x4 (&bb)[KW / 32], int p) {
            const int f = p % nfrag, q = p / nfrag;
            f32x4 tacc[MB];
#pragma unroll
            for (int b = 0; b < MB; ++b) tacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < KW / 32; ++s2) {
                const int kk = q * KP + wave * KW + 32 * s2 + 8 * g;  // within the slice
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    const u32x4 xv = *reinterpret_cast<const u32x4 *>(xs + (16 * b + l16) * XS + kk * 2);
                    tacc[b] = mfma16(bb[s2], xv, tacc[b]);
                }
            }
#pragma unroll
            for (int b = 0; b < MB; ++b) red[(wave * MB + b) * 64 + lane] = tacc[b];
            __syncthreads();
            if (wave == 0) {
                const int j = slice * (KS / KP) + q;
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    f32x4 t = red[b * 64 + lane];
#pragma unroll
                    for (int w = 1; w < 4; ++w) t += red[(w * MB + b) * 64 + lane];
                    const int m = 16 * b + l16;
                    bstore16<kDeviceCoherent>(rtp, (unsigned)((((j * nfrag + f) * a.M + m) * 16 + 4 * g) * 4) +
                                                       (m < a.M ? 0u : kOOB),
                                              __builtin_bit_cast(u32x4, t));
                }
            }
            __syncthreads();
        };
        // The first piece's B rows are the registers loaded before the Q
        // loads (this code path waits for nothing newer); later pieces load
        // their own.
        piece(bfirst, tn);
        for (int p = tn + a.pwg; p < a.pps; p += a.pwg) {
            u32x4 bb[KW / 32];
            load_b(bb, p);
            piece(bb, p);
        }
    }

    f32x4 acc[WNF][MB];
#pragma unroll
    for (int f = 0; f < WNF; ++f)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // K loop, fully unrolled: the loads of step s + D - 1 are issued before
    // step s is computed; scheduling barriers keep the compiler from sinking
    // them next to their uses.  Steps past `in` load zeros and add nothing.
#pragma unroll
    for (int s = 0; s < NSTEPS; ++s) {
        if (s + D - 1 < NSTEPS) load_q(qr[(s + D - 1) % D], s + D - 1);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 x0[MB], x1[MB];
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            const unsigned char *p = xs + (16 * b + l16) * XS + (64 * s + 16 * g) * 2;
            x0[b] = *reinterpret_cast<const u32x4 *>(p);
            x1[b] = *reinterpret_cast<const u32x4 *>(p + 16);
        }
#pragma unroll
        for (int f = 0; f < WNF; ++f) {
            u32x4 h0, h1;
            fp8x16_to_bf16x16(qr[s % D][f], h0, h1);
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                acc[f][b] = mfma16(h0, x0[b], acc[f][b]);
                acc[f][b] = mfma16(h1, x1[b], acc[f][b]);
            }
        }
        // Wave 0's piece stores were issued before the loads of step D - 1,
        // which this step has waited for: the stores are complete (device
        // scope) and the pieces can be announced.
        if (s == D - 1 && has_piece && wave == 0 && lane == 0) {
            for (int p = tn; p < a.pps; p += a.pwg) bump_u32(a.tflag);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // Lane holds acc[f][b][v] = (x dec(Q)^T)[m = 16 b + l16][n = nw + 16 f + 4 g + v]
    // summed over this slice.
    if (a.splits > 1) {
#pragma unroll
        for (int f = 0; f < WNF; ++f) {
            const int n = nw + f * 16 + 4 * g;
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const int m = b * 16 + l16;
                if (m >= a.M || n >= a.N) continue;
                if (a.y_vec) {  // out % 4 == 0: whole 16-byte groups
                    bstore16<kDeviceCoherent>(rp, (unsigned)(((int64_t)slice * a.M + m) * a.N + n) * 4u,
                                              __builtin_bit_cast(u32x4, acc[f][b]));
                } else {
                    float *dst = a.partials + ((int64_t)slice * a.M + m) * a.N + n;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (n + v < a.N)
                            __hip_atomic_store(dst + v, acc[f][b][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        // Every wave waits for its own stores (device scope), then the
        // barrier; only then does the counter move.
        wait_vmcnt<0>();
        __syncthreads();
        if (tid == 0) {
            // The first look at the T flag goes out together with the counter
            // update (neither waits for the other).
            const unsigned tf = poll_u32(a.tflag);
            const unsigned old = bump_u32(&a.cnt[tn]);
            tflag_sh = tf;
            is_last = old == (unsigned)(a.splits - 1) ? 1u : 0u;
        }
        __syncthreads();
        if (!is_last) return;
    }

    // Final work-group of the column tile.  Everything it reads goes out in
    // one round: the partial sums of the slices, the A rows and, if the T
    // flag already showed this launch's pieces complete, the T pieces.
    const unsigned tflag0 =
        a.splits > 1 ? tflag_sh : (a.r > 0 ? __builtin_amdgcn_readfirstlane(poll_u32(a.tflag)) : 0u);
    bool t_ready = a.r <= 0 || (int)(tflag0 - a.t_target) >= 0;

    constexpr int SB = 4;  // slices per batch of loads
    const unsigned pstride = (unsigned)a.M * (unsigned)a.N * 4u;
    auto load_batch = [&](f32x4 (&p)[SB][WNF][MB], int s0) {
#pragma unroll
        for (int u = 0; u < SB; ++u)
#pragma unroll
            for (int f = 0; f < WNF; ++f)
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    const int n = nw + f * 16 + 4 * g, m = b * 16 + l16;
                    const bool ok = s0 + u < a.splits && m < a.M && n < a.N;
                    p[u][f][b] = bload16f_dc(rp, (unsigned)(s0 + u) * pstride + (unsigned)(m * a.N + n) * 4u +
                                                     (ok ? 0u : kOOB));
                }
    };
    f32x4 pb[SB][WNF][MB];
    const bool vec_sum = a.splits > 1 && a.y_vec;
    if (vec_sum) load_batch(pb, 0);

    // T A^T runs over the padded rank 64 at a time (group h, two 32-rank
    // chunks c).  Lane holds A[n][64 h + 32 c + 8 g, +8) and, as bf16, T of
    // ranks 8 (g % 2) .. +8 of fragment 4 h + 2 c + g / 2 of row
    // m = 16 b + l16.  The float32 pieces of a group's four fragments are
    // staged in LDS (over the x slice, no longer read), jc K ranges at a
    // time, each read from memory once per work-group.
    const rsrc_t rtp = make_rsrc(a.tpart, (int64_t)a.t_splits * nfrag * a.M * 16 * 4);
    // A staged K range holds, for each of the 4 fragments, MB blocks of 64
    // units of 16 bytes (one load instruction each): unit 4 m + i of a
    // fragment is row m's ranks 4 i .. +4, units past 4 M read zero.
    constexpr int JU = 4 * MB * 64;  // units per staged K range
    const int jc = x_lds_bytes<MB, NSTEPS>() / (JU * 16);
    auto stage_t = [&](int h, int j0) {
        const int nj = a.t_splits - j0 < jc ? a.t_splits - j0 : jc;
        for (int i = wave; i < nj * 4 * MB; i += 4) {
            const int jj = i / (4 * MB), fr = (i / MB) % 4, k = i % MB, u = 64 * k + lane;
            const bool ok = u < 4 * a.M && 4 * h + fr < nfrag;
            const unsigned off = (unsigned)(((j0 + jj) * nfrag + 4 * h + fr) * a.M * 64 + u * 16) + (ok ? 0u : kOOB);
            bload16_lds<kDeviceCoherent>(rtp, xs + 1024 * i, off);
        }
    };
    if (a.r > 0) {
        // Every wave's last read of the x slice is behind it (with several
        // slices the barrier before the counter update already says so).
        if (a.splits <= 1) barrier_lds();
        if (t_ready) stage_t(0, 0);
    }

    // Sum of the slices, each element in slice order from zero.
    if (vec_sum) {
        f32x4 sum[WNF][MB];
#pragma unroll
        for (int f = 0; f < WNF; ++f)
#pragma unroll
            for (int b = 0; b < MB; ++b) sum[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0;;) {
#pragma unroll
            for (int u = 0; u < SB; ++u)
#pragma unroll
                for (int f = 0; f < WNF; ++f)
#pragma unroll
                    for (int b = 0; b < MB; ++b) sum[f][b] += pb[u][f][b];
            s0 += SB;
            if (s0 >= a.splits) break;
            load_batch(pb, s0);
        }
#pragma unroll
        for (int f = 0; f < WNF; ++f)
#pragma unroll
            for (int b = 0; b < MB; ++b) acc[f][b] = sum[f][b];
    } else if (a.splits > 1) {
        // Columns not in whole 16-byte groups: element loads, slice order.
#pragma unroll
        for (int f = 0; f < WNF; ++f) {
            const int n = nw + f * 16 + 4 * g;
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const int m = b * 16 + l16;
                f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
                if (m < a.M && n < a.N) {
                    for (int sl = 0; sl < a.splits; ++sl) {
                        const float *src = a.partials + ((int64_t)sl * a.M + m) * a.N + n;
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (n + v < a.N)
                                t[v] += __hip_atomic_load(src + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                acc[f][b] = t;
            }
        }
    }

#pragma unroll
    for (int f = 0; f < WNF; ++f)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[f][b] *= a.scale;

    if (a.r > 0) {
        if (!t_ready) {
            // The piece work-groups have the lowest ids and make their pieces
            // before they wait for anything; the bound only guards against a
            // broken dispatch-order assumption.  Each wave looks for itself.
            unsigned spins = 0;
            while ((int)(__builtin_amdgcn_readfirstlane(poll_u32(a.tflag)) - a.t_target) < 0 && ++spins < (1u << 26))
                __builtin_amdgcn_s_sleep(2);
            stage_t(0, 0);
        }
        for (int h = 0; h < a.r_pad / 64; ++h) {
            u32x4 af[2][WNF];
            if (h == 0) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int f = 0; f < WNF; ++f) af[c][f] = af0[c][f];
            } else {
                load_a(af, h);
            }
            // T over the K pieces in K order, rounded once to bf16: thread
            // tid sums the units tid + 256 i of the staged ranges and writes
            // them as bf16 to LDS (over `red`, same unit order), from where
            // every wave reads its operand.
            f32x4 ts[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i) ts[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int j0 = 0; j0 < a.t_splits; j0 += jc) {
                if (h > 0 || j0 > 0) {
                    barrier_lds_sync();  // every wave is done with the previous ranges
                    stage_t(h, j0);
                }
                wait_vmcnt<0>();
                barrier_lds();
                const int nj = a.t_splits - j0 < jc ? a.t_splits - j0 : jc;
                for (int jj = 0; jj < nj; ++jj) {
#pragma unroll
                    for (int i = 0; i < MB; ++i)
                        ts[i] += *reinterpret_cast<const f32x4 *>(xs + (jj * JU + tid + 256 * i) * 16);
                }
            }
            unsigned char *tb = reinterpret_cast<unsigned char *>(red);
#pragma unroll
            for (int i = 0; i < MB; ++i)
                *reinterpret_cast<u32x2 *>(tb + (tid + 256 * i) * 8) =
                    u32x2{pack_bf16x2(ts[i][0], ts[i][1]), pack_bf16x2(ts[i][2], ts[i][3])};
            barrier_lds_sync();
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    // Lane's operand: ranks 8 (g % 2) .. +8 of fragment
                    // 2 c + g / 2, row m = 16 b + l16 (rows past M hold zeros
                    // and only reach outputs that are not stored).
                    const u32x4 tf = *reinterpret_cast<const u32x4 *>(
                        tb + ((2 * c + (g >> 1)) * 64 * MB + 4 * (16 * b + l16) + 2 * (g & 1)) * 8);
#pragma unroll
                    for (int f = 0; f < WNF; ++f) acc[f][b] = mfma16(af[c][f], tf, acc[f][b]);
                }
            barrier_lds_sync();  // the next group's staging and bf16 T overwrite these
        }
    }

#pragma unroll
    for (int f = 0; f < WNF; ++f) {
        const int n = nw + f * 16 + 4 * g;
        if (n >= a.N) continue;
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            const int m = b * 16 + l16;
            if (m >= a.M) continue;
            const float o[4] = {acc[f][b][0] + bv[f][0], acc[f][b][1] + bv[f][1], acc[f][b][2] + bv[f][2],
                                acc[f][b][3] + bv[f][3]};
            store_out(a, m, n, o);
        }
    }
    if (a.splits > 1 && tid == 0) __hip_atomic_store(&a.cnt[tn], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MB, int NSTEPS>
hipError_t launch_sk(const SArgs &a, hipStream_t s) {
    if constexpr (x_lds_bytes<MB, NSTEPS>() + 4 * MB * 64 * 16 + 64 > LDS_MAX) {
        return hipErrorInvalidValue;
    } else {
        const int grid = a.tiles_n * a.splits;
        hipLaunchKernelGGL((skinny_kernel<MB, NSTEPS>), dim3(grid), dim3(SNT), 0, s, a);
        return hipGetLastError();
    }
}

template <int MB>
hipError_t launch_sk_steps(int k_slice, const SArgs &a, hipStream_t s) {
    switch (k_slice / 64) {
        case 8: return launch_sk<MB, 8>(a, s);
        case 16: return launch_sk<MB, 16>(a, s);
        case 32: return launch_sk<MB, 32>(a, s);
        case 64: return launch_sk<MB, 64>(a, s);
    }
    return hipErrorInvalidValue;
}

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

bool skinny_supports(int64_t M) { return M >= 1 && M <= SMAX_M; }

SkinnyPlan skinny_plan(int64_t M, int64_t K, int64_t N, int64_t r_pad, int64_t splits_hint) {
    SkinnyPlan pl{};
    pl.mb = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    pl.tiles_n = (int)cdiv64(N, SBN);
    // K slice (512 to 4096 elements): the x slice of 16 mb rows must fit in
    // LDS, and about one work-group per CU (or the hinted number of slices)
    // is wanted.
    const int64_t max_ks = 4096 / pl.mb;
    const int64_t want = splits_hint > 0 ? splits_hint : cdiv64(256, pl.tiles_n);
    const int64_t need = cdiv64(K, want < 1 ? 1 : want);
    int64_t ks = 512;
    while (ks < need && ks < max_ks) ks *= 2;
    pl.k_slice = (int)ks;
    pl.splits = (int)cdiv64(K, ks);
    // T pieces: 16 ranks over KP elements of a slice each (KP = 4 x 256, or
    // the whole slice when that is shorter); the first pwg work-groups of
    // every slice compute them.
    pl.groups = (int)(r_pad / 16);
    const int64_t kp = ks < 1024 ? ks : 1024;
    pl.t_kslice = (int)kp;
    pl.pps = (int)(pl.groups * (ks / kp));
    pl.pwg = pl.pps < pl.tiles_n ? pl.pps : pl.tiles_n;
    pl.t_splits = (int)(pl.splits * (ks / kp));
    pl.producers = r_pad > 0 ? pl.pwg * pl.splits : 0;  // work-groups that compute pieces
    return pl;
}

int64_t skinny_sync_words(const SkinnyPlan &pl) { return (int64_t)pl.tiles_n + 1; }

bool skinny_shape_ok(int64_t M, int64_t K, int64_t N, int64_t r_pad, const SkinnyPlan &pl, int64_t ldx) {
    // Every buffer descriptor must stay below 2^31 bytes.
    const int64_t lim = (int64_t)1 << 31;
    // The piece work-groups must all be resident at once (at most one per CU).
    return (int64_t)SBN * K < lim && M * ldx * 2 < lim && r_pad * K * 2 < lim && (int64_t)SBN * r_pad * 2 < lim &&
           (int64_t)pl.splits * M * N * 4 < lim && (int64_t)pl.t_splits * M * r_pad * 4 < lim && N * 2 < lim &&
           K < lim && (int64_t)pl.tiles_n * pl.splits < lim && pl.producers <= 256;
}

hipError_t launch_skinny(const SkinnyProblem &p, const void *a_eff, hipStream_t s) {
    const SkinnyPlan &pl = p.plan;
    if (!p.sync || (pl.splits > 1 && !p.partials) || (p.r > 0 && !p.t_part)) return hipErrorInvalidValue;
    SArgs a{};
    a.x = (const unsigned char *)p.x;
    a.ldx = (int)p.ldx;
    a.B = (const unsigned char *)p.B;
    a.Q = (const unsigned char *)p.Q;
    a.A = (const unsigned char *)a_eff;
    a.bias = (const unsigned char *)p.bias;
    a.y = p.y;
    a.partials = p.partials;
    a.tpart = p.t_part;
    a.scale = p.scale;
    a.M = (int)p.M;
    a.K = (int)p.K;
    a.N = (int)p.N;
    a.r = (int)p.r;
    a.r_pad = (int)p.r_pad;
    a.lda = a_eff == p.A ? (int)p.r : (int)p.r_pad;
    a.splits = pl.splits;
    a.tiles_n = pl.tiles_n;
    a.t_splits = pl.t_splits;
    a.pps = pl.pps;
    a.pwg = p.r > 0 ? pl.pwg : 0;
    a.cnt = p.sync;
    a.tflag = p.sync + pl.tiles_n;
    a.t_target = p.t_target;
    a.y_vec = (p.N % 4 == 0) && ((uintptr_t)p.y % 16 == 0) && ((uintptr_t)p.partials % 16 == 0);
    a.out_f32 = p.out_f32;
    a.gelu = p.gelu;
    switch (pl.mb) {
        case 1: return launch_sk_steps<1>(pl.k_slice, a, s);
        case 2: return launch_sk_steps<2>(pl.k_slice, a, s);
        case 4: return launch_sk_steps<4>(pl.k_slice, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ll
