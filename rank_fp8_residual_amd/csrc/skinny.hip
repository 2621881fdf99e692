// Skinny-M (HBM-bound) path of the fused LiteLinear forward on gfx950.
//
// The forward (LiteLinear README, page "moonmath-ai/LiteLinear", equation in
// the introduction):  y = (x B^T) A^T + scale * (x dec(Q)^T) + bias.
//
// With few rows the time is the time to stream Q (out * in bytes) from HBM
// once, so the launch is organised around that stream.  Two kernels:
//
// skinny_fullk_kernel (up to 16 rows, 2048 < in <= 8192, enough columns to
// fill the chip): every work-group owns 32 columns over all of K, streamed
// through a ring of LDS stages, and no partial sums leave it; described at
// the kernel.
//
// skinny_kernel (every other shape up to 64 rows), split over K:
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
//     at zero; the T flag counts this launch's pieces, and the last final
//     work-group to finish reading them (a second counter) sets both back to
//     zero, so every launch waits for the same constant target and a
//     captured launch replays correctly.
// Only final work-groups wait, and only for T pieces.  The piece work-groups
// have the lowest ids (at most one per CU), so they are dispatched first and
// compute their pieces before waiting for anything: the waits always end.
// They are bounded all the same; one that gives up sets the error word that
// the host reports as a status.
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
constexpr int XPAD = 8;            // bf16 of padding per LDS row of x
constexpr int LDS_MAX = 160 * 1024;

struct SArgs {
    const unsigned char *x, *B, *Q, *A, *bias;
    void *y;
    float *partials;     // [splits, M, N]
    unsigned *cnt;       // [tiles_n] K slices done per column tile
    unsigned *tflag;     // T pieces finished in this launch
    unsigned *fdone;     // final work-groups done reading the T pieces
    unsigned *err;       // host-visible error word, set when a bounded wait gives up
    unsigned t_target;   // tflag value meaning "this launch's T is complete"
    unsigned wait_limit; // polls before a wait gives up
    float *tpart;        // T pieces, float32 [t_splits, r_pad / 16, M, 16]
    unsigned long long *gen;  // all-of-K kernel: [0] T pieces made, [32 (1 + x)]
                              // work-groups c % 32 == x started (never reset)
    float scale;
    int M, K, N, r, r_pad, lda, splits, tiles_n, t_splits;
    int ldx;             // elements between rows of x (>= K)
    int pps;             // T pieces per K slice (16 ranks x a part of the slice each)
    int pwg;             // work-groups of a slice that compute pieces (lowest ids)
    bool y_vec, out_f32, gelu;
    // Gated epilogue: Q, A and bias hold 2F rows (hidden, then gate), y is
    // [M, F] = hidden * GELU_erf(gate).  A work-group's 128 columns of the
    // products are 64 output columns twice: wave w's fragment 0 is hidden
    // columns [64 tn + 16 w, +16), fragment 1 the gate of the same columns.
    // N is then the products' column count (tiles_n x 128, the partial
    // sums' row length) and NO = F the output's; otherwise NO = N.
    bool glu;
    int F, NO;
};

// ------------------------------------------------------------ output tiles

// y[m][n .. n + 3] = y (past NO dropped), through the activation option.
__device__ __forceinline__ void store_out(const SArgs &a, int m, int n, const float (&y)[4]) {
    float o[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) o[v] = a.gelu ? gelu_tanh(y[v]) : y[v];
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

// --------------------------------------------------- per-lane coordinates

// Where a lane sits: its wave, its 16-row group and 4-column group of the
// matrix-core tiles, the work-group's K slice and column tile (the pwg
// piece work-groups of every slice come first), the wave's output columns
// and, with the gated epilogue, its first output column.
struct SLane {
    int tid, lane, wave, l16, g;
    int slice, tn, n0, nw, c0, rows_n;
    bool piece_wg;
};

__device__ __forceinline__ SLane skinny_lane(const SArgs &a) {
    SLane L;
    L.tid = (int)threadIdx.x;
    L.lane = L.tid & 63;
    L.wave = L.tid >> 6;
    L.l16 = L.lane & 15;
    L.g = L.lane >> 4;
    const int c = (int)blockIdx.x;
    L.piece_wg = c < a.pwg * a.splits;
    if (L.piece_wg) {
        L.slice = c / a.pwg;
        L.tn = c - L.slice * a.pwg;
    } else {
        const int c2 = c - a.pwg * a.splits, rest = a.tiles_n - a.pwg;
        L.slice = c2 / rest;
        L.tn = a.pwg + (c2 - L.slice * rest);
    }
    L.n0 = L.tn * SBN;
    L.nw = L.n0 + L.wave * (WNF * 16);
    L.rows_n = (a.N - L.n0) < SBN ? (a.N - L.n0) : SBN;
    L.c0 = L.tn * (SBN / 2) + L.wave * 16;
    return L;
}

// Row of Q and A, relative to the descriptors of q_rsrc / a_rsrc, behind
// row l of fragment f of the work-group's column group w (32 columns; a
// wave's columns in the epilogue); kNoRow where there is none.  With the
// gated epilogue fragment 0 is the hidden half and fragment 1 the gate of
// output columns [64 tn + 16 w, +16).
constexpr unsigned kNoRow = 0x7FFFFFFFu;
__device__ __forceinline__ unsigned q_row(const SArgs &a, int tn, int w, int f, int l) {
    if (a.glu) {
        const int c = tn * (SBN / 2) + 16 * w + l;
        return c < a.F ? (unsigned)(f * a.F + c) : kNoRow;
    }
    return (unsigned)(w * (WNF * 16) + 16 * f + l);
}

__device__ __forceinline__ rsrc_t q_rsrc(const SArgs &a, const SLane &L) {
    return a.glu ? make_rsrc(a.Q, (int64_t)2 * a.F * a.K) : make_rsrc(a.Q + (int64_t)L.n0 * a.K, (int64_t)L.rows_n * a.K);
}

__device__ __forceinline__ rsrc_t a_rsrc(const SArgs &a, const SLane &L) {
    return a.glu ? make_rsrc(a.A, (int64_t)2 * a.F * a.lda * 2)
                 : make_rsrc(a.A + (int64_t)L.n0 * a.lda * 2, (int64_t)L.rows_n * a.lda * 2);
}

// Bias of the lane's output columns (past N and a missing bias read as zero).
__device__ __forceinline__ void load_bias(const SArgs &a, const SLane &L, float (&bv)[WNF][4]) {
    const rsrc_t rb = make_rsrc(a.bias, a.bias ? (int64_t)(a.glu ? 2 * a.F : a.N) * 2 : 0);
#pragma unroll
    for (int f = 0; f < WNF; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (a.glu) {
                const int cc = L.c0 + 4 * L.g + v;
                bv[f][v] = bload_bf16(rb, (unsigned)(f * a.F + cc) + (cc < a.F ? 0u : kOOB / 2));
            } else {
                bv[f][v] = bload_bf16(rb, (unsigned)(L.nw + 16 * f + 4 * L.g + v));
            }
        }
}

// Ranks [64 h, +64) of the lane's A rows: A[row][64 h + 32 c + 8 g, +8).
__device__ __forceinline__ void load_a(const SArgs &a, const SLane &L, rsrc_t ra, u32x4 (&af)[2][WNF], int h) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int f = 0; f < WNF; ++f) {
            const int ka = 64 * h + 32 * c + 8 * L.g;
            const unsigned row = q_row(a, L.tn, L.wave, f, L.l16);
            af[c][f] = bload16(ra, (row * (unsigned)a.lda + (unsigned)ka) * 2u + (ka < a.lda && row != kNoRow ? 0u : kOOB));
        }
}

// ------------------------------------------------------- the common tail
//
// After the residual product of its slice: lane holds acc[f][b][v] =
// (x dec(Q)^T)[m = 16 b + l16][n = nw + 16 f + 4 g + v] over the slice.
// With several slices the partial sums go out and only the column tile's
// last work-group goes on; that one adds the slices, scales, adds T A^T and
// the bias and stores y.  `stage` (STAGE bytes of LDS that no wave reads any
// more) holds the T pieces on their way in; `red` (at least 2 KiB x MB)
// holds T as bf16.
// bv and af0 hold the bias of the lane's columns and the first 64 ranks of
// its A rows, requested by the kernel long before.
template <int MB, int STAGE>
__device__ __forceinline__ void skinny_tail(const SArgs &a, const SLane &L, f32x4 (&acc)[WNF][MB],
                                            const float (&bv)[WNF][4], const u32x4 (&af0)[2][WNF],
                                            unsigned char *stage, f32x4 *red, unsigned &is_last,
                                            unsigned &tflag_sh) {
    const int tid = L.tid, lane = L.lane, wave = L.wave, l16 = L.l16, g = L.g, tn = L.tn, nw = L.nw;
    const int nfrag = a.r_pad / 16;
    const rsrc_t rp = make_rsrc(a.partials, a.splits > 1 ? (int64_t)a.splits * a.M * a.N * 4 : 0);
    if (a.splits > 1) {
#pragma unroll
        for (int f = 0; f < WNF; ++f) {
            const int n = nw + f * 16 + 4 * g;
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const int m = b * 16 + l16;
                if (m >= a.M || n >= a.N) continue;
                if (a.y_vec) {  // out % 4 == 0: whole 16-byte groups
                    bstore16<kDeviceCoherent>(rp, (unsigned)(((int64_t)L.slice * a.M + m) * a.N + n) * 4u,
                                              __builtin_bit_cast(u32x4, acc[f][b]));
                } else {
                    float *dst = a.partials + ((int64_t)L.slice * a.M + m) * a.N + n;
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
    bool t_ready = a.r <= 0 || tflag0 >= a.t_target;

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
    // staged in LDS, jc K ranges at a time, each read from memory once per
    // work-group.
    const rsrc_t rtp = make_rsrc(a.tpart, (int64_t)a.t_splits * nfrag * a.M * 16 * 4);
    // A staged K range holds, for each of the 4 fragments, MB blocks of 64
    // units of 16 bytes (one load instruction each): unit 4 m + i of a
    // fragment is row m's ranks 4 i .. +4, units past 4 M read zero.
    constexpr int JU = 4 * MB * 64;  // units per staged K range
    constexpr int jc = STAGE / (JU * 16);
    static_assert(jc >= 1, "T staging area");
    auto stage_t = [&](int h, int j0) {
        const int nj = a.t_splits - j0 < jc ? a.t_splits - j0 : jc;
        for (int i = wave; i < nj * 4 * MB; i += 4) {
            const int jj = i / (4 * MB), fr = (i / MB) % 4, k = i % MB, u = 64 * k + lane;
            const bool ok = u < 4 * a.M && 4 * h + fr < nfrag;
            const unsigned off = (unsigned)(((j0 + jj) * nfrag + 4 * h + fr) * a.M * 64 + u * 16) + (ok ? 0u : kOOB);
            bload16_lds<kDeviceCoherent>(rtp, stage + 1024 * i, off);
        }
    };
    if (a.r > 0) {
        // Every wave's last read of the staging area is behind it (with
        // several slices the barrier before the counter update already says
        // so).
        if (a.splits <= 1) barrier_lds_sync();
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
            // broken dispatch-order assumption (reported through the error
            // word).  Each wave looks for itself.
            unsigned spins = 0;
            while (__builtin_amdgcn_readfirstlane(poll_u32(a.tflag)) < a.t_target) {
                if (++spins >= a.wait_limit) {
                    if (lane == 0) report_wait_timeout(a.err);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            stage_t(0, 0);
        }
        const rsrc_t ra = a_rsrc(a, L);
        for (int h = 0; h < a.r_pad / 64; ++h) {
            u32x4 af[2][WNF];
            if (h == 0) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int f = 0; f < WNF; ++f) af[c][f] = af0[c][f];
            } else {
                load_a(a, L, ra, af, h);
            }
            // T over the K pieces in K order, rounded once to bf16: thread
            // tid sums the units tid + 256 i of the staged ranges and writes
            // them as bf16 to LDS (`red`, same unit order), from where every
            // wave reads its operand.
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
                        ts[i] += *reinterpret_cast<const f32x4 *>(stage + (jj * JU + tid + 256 * i) * 16);
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
        // Every T piece this work-group reads has landed (the staging waits
        // above); the launch's last final work-group restarts both counters.
        if (tid == 0 && bump_u32(a.fdone) == (unsigned)(a.tiles_n - 1)) {
            __hip_atomic_store(a.tflag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.fdone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    if (a.glu) {
        // y = hidden * GELU_erf(gate): fragment 0 holds the hidden columns
        // c0 + 4 g .. of this lane, fragment 1 their gate
        const int n = L.c0 + 4 * g;
        if (n < a.F) {
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const int m = b * 16 + l16;
                if (m >= a.M) continue;
                float o[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = (acc[0][b][v] + bv[0][v]) * gelu_erf(acc[1][b][v] + bv[1][v]);
                store_out(a, m, n, o);
            }
        }
    } else {
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
    }
    if (a.splits > 1 && tid == 0) __hip_atomic_store(&a.cnt[tn], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sixteen residual codes -> two bf16 operands of 8 (QF: 0 e4m3fn, 1
// e4m3fnuz: the halving conversion, and the fix-up of the three exceptional
// codes in the rare lane that holds one).
template <int QF>
__device__ __forceinline__ void q16_to_bf16(u32x4 q, u32x4 &h0, u32x4 &h1) {
    if constexpr (QF == 0) {
        fp8x16_to_bf16x16(q, h0, h1);
    } else {
        u32x2 c[4] = {q8x4_to_bf16x4<1>(q.x), q8x4_to_bf16x4<1>(q.y), q8x4_to_bf16x4<1>(q.z), q8x4_to_bf16x4<1>(q.w)};
        const unsigned sp = fnuz_special_or(fnuz_special_or(fnuz_special_or(fnuz_special_or(0u, q.x), q.y), q.z), q.w);
        if (fnuz_any_special(sp)) {
            c[0] = fnuz_patch(q.x, c[0]);
            c[1] = fnuz_patch(q.y, c[1]);
            c[2] = fnuz_patch(q.z, c[2]);
            c[3] = fnuz_patch(q.w, c[3]);
        }
        h0 = u32x4{c[0].x, c[0].y, c[1].x, c[1].y};
        h1 = u32x4{c[2].x, c[2].y, c[3].x, c[3].y};
    }
}

// ------------------------------------------- 17 to 64 rows: x in LDS

// MB row blocks of 16, K slice of NSTEPS x 64; QF: residual codes in
// e4m3fn (0) or e4m3fnuz (1).
template <int MB, int NSTEPS, int QF>
__global__ void __launch_bounds__(SNT) skinny_kernel(SArgs a) {
    constexpr int KS = NSTEPS * 64;            // K elements per slice
    constexpr int XS = (KS + XPAD) * 2;        // LDS bytes per row of x
    constexpr int D = DEPTH < NSTEPS ? DEPTH : NSTEPS;
    constexpr int KW = t_kwave<NSTEPS>();      // K of a T piece per wave
    constexpr int KP = 4 * KW;                 // K of a T piece
    __shared__ __attribute__((aligned(16))) unsigned char xs[x_lds_bytes<MB, NSTEPS>()];
    __shared__ f32x4 red[4 * MB * 64];
    __shared__ unsigned is_last, tflag_sh;

    const SLane L = skinny_lane(a);
    const int lane = L.lane, wave = L.wave, l16 = L.l16, g = L.g, tn = L.tn, slice = L.slice;
    const int kb = slice * KS;

    // Uniform descriptors (built here so they stay in scalar registers).
    const rsrc_t rq = q_rsrc(a, L);
    const rsrc_t rx = make_rsrc(a.x, (int64_t)a.M * a.ldx * 2);

    // Bias and the first 64 ranks of the lane's A rows, requested up front:
    // A is read from HBM for the first time, and only a final work-group
    // (any work-group may be one) uses it, after its Q stream.
    float bv[WNF][4];
    load_bias(a, L, bv);
    u32x4 af0[2][WNF];
    if (a.r > 0) load_a(a, L, a_rsrc(a, L), af0, 0);

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
    const bool has_piece = L.piece_wg && a.r > 0;
    if (has_piece) load_b(bfirst, tn);

    // Q: lane holds codes [k + 16 g, +16) of row nw + 16 f + l16 (of row
    // q_row(f) with the gated epilogue).
    unsigned qoff[WNF];
#pragma unroll
    for (int f = 0; f < WNF; ++f) {
        const unsigned row = q_row(a, tn, wave, f, l16);
        qoff[f] = row == kNoRow ? kOOB : row * (unsigned)a.K;
    }
    auto load_q = [&](u32x4 (&q)[WNF], int s) {
        const int k = kb + 64 * s + 16 * g;
        const unsigned oob = k < a.K ? 0u : kOOB;
#pragma unroll
        for (int f = 0; f < WNF; ++f) q[f] = bload16_nt(rq, qoff[f] + (unsigned)k + oob);
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
            q16_to_bf16<QF>(qr[s % D][f], h0, h1);
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

    skinny_tail<MB, x_lds_bytes<MB, NSTEPS>()>(a, L, acc, bv, af0, xs, red, is_last, tflag_sh);
}

// ------------------------- up to 16 rows, wide outputs: all of K per work-group
//
// Each work-group owns 32 product columns (two 16-row fragments of Q) over
// all of K, so no partial sums leave it: wave w streams K quarter w of those
// rows through a private ring of NB LDS stages, and the four quarters are
// added in wave order at the end.  A stage is 32 rows (the two 16-row
// fragments) x 256 codes, moved by 8 direct-to-LDS loads that each cover 4
// rows x 256 bytes (loading Q straight into matrix-core operand registers
// makes every load instruction touch 16 rows x 64 bytes, which measured a
// quarter slower on the same bytes); lane l of a load lands at slot l % 16
// of its row and fetches 16-byte chunk (l % 16) ^ row, so that the operand
// reads afterwards (16 rows, one chunk each) hit 16 distinct 16-byte bank
// groups.  The x chunk of each stage (16 rows x 256, from L2) is loaded into
// registers with the stage.
//
// Each work-group walks its stages in a rotated order (its own first stage),
// which spreads the work-groups that run at the same time over different
// lines of x in L2 and different channels of Q in HBM: with every
// work-group on the same stage together, the x loads measured a sixth of
// the kernel's time.
//
// T = x B^T comes in pieces: piece (f, ph) is ranks [16 f, +16) over K
// phase ph (the 256-element chunks [ph SPP, +SPP) of every wave's quarter),
// made by the work-group with id ph * (r_pad / 16) + f, the lowest ids.  A
// piece work-group starts its rotation at chunk ph SPP, so the piece takes
// its x from the registers of its first SPP stages; it loads only its B
// rows, makes the piece before it refills the ring after stage SPP - 1 and
// announces it once the stores are complete.  Every work-group waits for all
// pieces (long since made) at its end, stages them in LDS and adds them in
// phase order.
//
// The hand-over counts with 64-bit counters that only grow, so nothing has
// to be reset at the end of a launch (and a captured launch replays
// correctly): gen[0] counts pieces made over all launches on the workspace,
// and 32 ticket counters (gen[32 (1 + x)], each in its own 256 bytes) count
// the work-groups c with c % 32 == x started.  A work-group's ticket, taken
// first thing, is L n_x + i for launch L (launches on one workspace run one
// after another; n_x work-groups per launch share the counter), so this
// launch's pieces are complete once gen[0] reaches (L + 1) pps.  The ticket
// is taken behind the first ring loads, and read once a later stage's wait
// covers it; spread over 32 counters, the tickets' atomics do not hold up
// those stages (on one counter all 256 queue up for microseconds).
//
// NQ: stages per wave (K quarter = 256 NQ; 4 or 8).
template <int NQ, int QF>
__global__ void __launch_bounds__(SNT) skinny_fullk_kernel(SArgs a) {
    constexpr int KQ = 256 * NQ;
    constexpr int NB = 4;               // ring slots per wave
    constexpr int STB = 32 * 256;       // bytes per stage
    constexpr int RING = 4 * STB;
    constexpr int PH = NQ;              // K phases of T (one stage each: the B
                                        // operands of two would cost the
                                        // registers that keep the waits exact)
    constexpr int SPP = NQ / PH;        // stages per phase
    constexpr int NP = 8 * SPP;         // B operands per lane of a piece
    static_assert(NQ == 4 || NQ == 8, "stages per wave");
    static_assert(PH * 4 * 1024 <= RING, "T pieces of a 64-rank group fit one ring array");
    __shared__ __attribute__((aligned(16))) unsigned char ring0[RING], ring1[RING], ring2[RING], ring3[RING];
    __shared__ __attribute__((aligned(16))) unsigned char tb[16 * 128];  // a 64-rank group of T as bf16 [m][64]
    __shared__ f32x4 red[4 * 64];
    __shared__ unsigned tflag_sh;

    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
    const int c = (int)blockIdx.x;
    const int kq = wave * KQ;
    const int nfrag = a.r_pad / 16;
    unsigned long long ticket = 0;
    const bool has_piece = a.r > 0 && c < a.pps;
    const int pf = has_piece ? c % nfrag : 0, pph = has_piece ? c / nfrag : 0;
    // the first stage of this work-group's rotation
    const int rot = has_piece ? pph * SPP : c % NQ;

    // Rows of Q and A behind row l of fragment f (kNoRow: none).  Plain: the
    // product columns [32 c, +32); gated: output columns [16 c, +16), hidden
    // rows then gate rows.
    const int n0 = 32 * c;
    const int rows_n = a.N - n0 < 32 ? a.N - n0 : 32;
    auto row_of = [&](int f, int l) -> unsigned {
        if (a.glu) {
            const int cc = 16 * c + l;
            return cc < a.F ? (unsigned)(f * a.F + cc) : kNoRow;
        }
        return (unsigned)(16 * f + l);
    };
    const rsrc_t rq = a.glu ? make_rsrc(a.Q, (int64_t)2 * a.F * a.K) : make_rsrc(a.Q + (int64_t)n0 * a.K, (int64_t)rows_n * a.K);
    const rsrc_t ra = a.glu ? make_rsrc(a.A, (int64_t)2 * a.F * a.lda * 2)
                            : make_rsrc(a.A + (int64_t)n0 * a.lda * 2, (int64_t)rows_n * a.lda * 2);
    const rsrc_t rb = make_rsrc(a.bias, a.bias ? (int64_t)(a.glu ? 2 * a.F : a.N) * 2 : 0);
    const rsrc_t rx = make_rsrc(a.x, (int64_t)a.M * a.ldx * 2);
    const rsrc_t rbm = make_rsrc(a.B, (int64_t)a.r * a.K * 2);

    // x chunk j of K position k: x[l16][k + 64 (j / 2) + 16 g + 8 (j % 2), +8)
    // (rows past M and columns past `in` read zero); the same layout for B.
    auto xoff = [&](int k, int j) -> unsigned {
        const int kk = k + 64 * (j >> 1) + 16 * g + 8 * (j & 1);
        return ((unsigned)l16 * (unsigned)a.ldx + (unsigned)kk) * 2u + (kk < a.K ? 0u : kOOB);
    };

    // The first loads: the bias and the first 64 ranks of the A rows (for
    // the epilogue), and a piece work-group's B rows (the rest of the
    // work-groups issue the same loads out of range, which keeps the wait
    // counts constant).
    float bv[WNF][4];
#pragma unroll
    for (int f = 0; f < WNF; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (a.glu) {
                const int cc = 16 * c + 4 * g + v;
                bv[f][v] = bload_bf16(rb, (unsigned)(f * a.F + cc) + (cc < a.F ? 0u : kOOB / 2));
            } else {
                bv[f][v] = bload_bf16(rb, (unsigned)(n0 + 16 * f + 4 * g + v));
            }
        }
    u32x4 af0[2][WNF];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int f = 0; f < WNF; ++f) {
            const int ka = 32 * cc + 8 * g;
            const unsigned row = row_of(f, l16);
            af0[cc][f] = bload16(ra, (row * (unsigned)a.lda + (unsigned)ka) * 2u + (ka < a.lda && row != kNoRow ? 0u : kOOB));
        }
    u32x4 pb[NP];
    {
        const int kp = kq + 256 * SPP * pph;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int kk = kp + 256 * (j / 8) + 64 * ((j % 8) >> 1) + 16 * g + 8 * (j & 1);
            pb[j] = bload16(rbm, ((unsigned)(16 * pf + l16) * (unsigned)a.K + (unsigned)kk) * 2u +
                                     (has_piece && kk < a.K ? 0u : kOOB));
        }
    }

    // The ring, one LDS array per slot (each holding that slot of every
    // wave): as distinct objects the compiler can tell that reading one slot
    // does not wait for the direct-to-LDS loads still filling the others.
    // Stage s of this wave is K [kq + 256 ((s + rot) % NQ), +256) of the 32
    // rows, 8 direct-to-LDS loads of 4 rows x 256 bytes, then the 8 x
    // operands of the same K.
    auto slot_ptr = [&](int slot) -> unsigned char * {
        unsigned char *r = slot == 0 ? ring0 : (slot == 1 ? ring1 : (slot == 2 ? ring2 : ring3));
        return r + wave * STB;
    };
    const int lr = lane >> 4, ls = lane & 15;
    u32x4 xr[NQ][8];
    auto load_stage = [&](int slot, int s) {
        const int k0 = kq + 256 * ((s + rot) % NQ);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int R = 4 * i + lr, l = R & 15;
            const int k = k0 + 16 * (ls ^ l);
            const unsigned row = row_of(R >> 4, l);
            const unsigned off = row == kNoRow || k >= a.K ? kOOB : row * (unsigned)a.K + (unsigned)k;
            bload16_lds<kNonTemporal>(rq, slot_ptr(slot) + 1024 * i, off);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) xr[s][j] = bload16(rx, xoff(k0, j));
        // (the wait counts assume the loads go out in this order, stage by
        // stage)
        __builtin_amdgcn_sched_barrier(0);
    };
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < NB; ++s) load_stage(s, s);

    const rsrc_t rtp = make_rsrc(a.tpart, (int64_t)PH * nfrag * a.M * 16 * 4);
    f32x4 acc[WNF];
#pragma unroll
    for (int f = 0; f < WNF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    unsigned long long made0 = 0, target = 0;
    // this launch's piece count, from the ticket (read in a middle stage,
    // when the ticket's atomic has long returned)
    auto u64_uniform = [](unsigned long long v) {
        return ((unsigned long long)__builtin_amdgcn_readfirstlane((unsigned)(v >> 32)) << 32) |
               (unsigned)__builtin_amdgcn_readfirstlane((unsigned)v);
    };

    // The piece's store goes out in stage SPP - 1, after the loads of stage
    // SPP + NB - 2 and before those of stage SPP + NB - 1: one operation more
    // than the wait for stage SPP + NB - 2 leaves in flight, so that wait
    // covers it (in wave 0, the one that stores).
    constexpr int BUMP_AT = SPP + NB - 2 < NQ - 1 ? SPP + NB - 2 : NQ - 1;
    // The ticket goes out in stage 0 right after the loads of stage NB (if
    // any): the wait for stage NB covers it (one operation more than it
    // leaves in flight), or the last stage's wait for everything.
    constexpr int TICKET_READ = NB < NQ ? NB : NQ - 1;
    auto step = [&](auto S) {
        constexpr int s = decltype(S)::value;
        constexpr int later = 16 * ((s + NB < NQ ? s + NB : NQ) - s - 1);
        wait_vmcnt<later>();
        asm volatile("" ::: "memory");
        if (s == BUMP_AT && has_piece && wave == 0 && lane == 0)
            __hip_atomic_fetch_add(a.gen, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (s == TICKET_READ) {
            const unsigned nx = (gridDim.x - (unsigned)(c % 32) + 31) / 32;  // work-groups on this ticket counter
            target = (u64_uniform(ticket) / nx + 1) * (unsigned long long)a.pps + a.t_target;
        }
        // wave 0's look at the piece count two stages before the end, used
        // afterwards
        if constexpr (s == NQ - 2) {
            if (wave == 0 && a.r > 0) made0 = __hip_atomic_load(a.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const unsigned char *st = slot_ptr(s % NB);
        u32x4 q[WNF][4];
#pragma unroll
        for (int f = 0; f < WNF; ++f)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                q[f][t] = *reinterpret_cast<const u32x4 *>(st + (16 * f + l16) * 256 + (((4 * t + g) ^ l16) << 4));
        wait_lgkmcnt0();
        asm volatile("" ::: "memory");
        if constexpr (s == SPP - 1) {
            if (has_piece) {
                // piece (pf, pph) from the x of stages 0 .. SPP - 1 (chunks
                // pph SPP ..): the four waves' quarters added in wave order
                // through LDS by wave 0, stored as float32 [pph][pf][m][16]
                f32x4 tacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < SPP; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j) tacc = mfma16(pb[8 * i + j], xr[i][j], tacc);
                red[wave * 64 + lane] = tacc;
                barrier_lds_sync();
                if (wave == 0) {
                    f32x4 t = red[lane];
#pragma unroll
                    for (int w = 1; w < 4; ++w) t += red[w * 64 + lane];
                    bstore16<kDeviceCoherent>(rtp, (unsigned)((((pph * nfrag + pf) * a.M + l16) * 16 + 4 * g) * 4) +
                                                       (l16 < a.M ? 0u : kOOB),
                                              __builtin_bit_cast(u32x4, t));
                }
                barrier_lds_sync();
            }
        }
        if constexpr (s + NB < NQ) load_stage(s % NB, s + NB);
        __builtin_amdgcn_sched_barrier(0);
        // the ticket (wave 0, lane 0), right behind the loads of stage NB
        if constexpr (s == 0) {
            if (a.r > 0 && tid == 0)
                ticket = __hip_atomic_fetch_add(a.gen + 32 * (1 + c % 32), 1ull, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < WNF; ++f)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                u32x4 h0, h1;
                q16_to_bf16<QF>(q[f][t], h0, h1);
                acc[f] = mfma16(h0, xr[s][2 * t], acc[f]);
                acc[f] = mfma16(h1, xr[s][2 * t + 1], acc[f]);
            }
        __builtin_amdgcn_sched_barrier(0);
    };
    static_for<0, NQ>(step);

    // The four K quarters, added in wave order by wave 0.
#pragma unroll
    for (int f = 0; f < WNF; ++f) *reinterpret_cast<f32x4 *>(slot_ptr(0) + f * 1024 + lane * 16) = acc[f];
    if (a.r > 0 && wave == 0) {
        // T: wave 0 waits for this launch's pieces (the count was read two
        // stages ago; the pieces are normally long complete); after the
        // barrier each wave stages its phase of each 64-rank group.
        if (u64_uniform(made0) < target) {
            // (polled every few hundred cycles: the counter shares its
            // memory channel with the Q stream of the work-groups still
            // running, and hundreds of close polls slow both)
            unsigned spins = 0;
            while (u64_uniform(__hip_atomic_load(a.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < target) {
                if (++spins >= a.wait_limit) {
                    if (lane == 0) report_wait_timeout(a.err);
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
        }
    }
    barrier_lds_sync();
    // (ring1, free since its last stage, holds the staged pieces): each wave
    // stages phases wave, wave + 4, .. of fragments 4 h .. 4 h + 3, 1 KiB each
    unsigned char *const tst = ring1;
    auto stage_t = [&](int h) {
#pragma unroll
        for (int ph = wave; ph < PH; ph += 4)
#pragma unroll
            for (int fr = 0; fr < 4; ++fr) {
                const bool ok = 4 * h + fr < nfrag && lane < 4 * a.M;
                bload16_lds<kDeviceCoherent>(rtp, tst + (ph * 4 + fr) * 1024,
                                             (unsigned)(((ph * nfrag + 4 * h + fr) * a.M * 16) * 4 + lane * 16) +
                                                 (ok ? 0u : kOOB));
            }
    };
    if (a.r > 0) stage_t(0);  // in flight while wave 0 adds the quarters
    f32x4 sum[WNF];
    if (wave == 0) {
#pragma unroll
        for (int f = 0; f < WNF; ++f) {
            sum[f] = *reinterpret_cast<const f32x4 *>(ring0 + f * 1024 + lane * 16);
#pragma unroll
            for (int v = 1; v < 4; ++v) sum[f] += *reinterpret_cast<const f32x4 *>(ring0 + v * STB + f * 1024 + lane * 16);
            sum[f] *= a.scale;
        }
    }
    for (int h = 0; h < a.r_pad / 64; ++h) {
        wait_vmcnt<0>();
        barrier_lds();
        if (wave == 0) {
            // lane (fr = g, m = l16): T[m][16 fr .. +16) over the phases in
            // order, rounded once to bf16
            f32x4 t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ph = 0; ph < PH; ++ph)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    t[i] += *reinterpret_cast<const f32x4 *>(tst + (ph * 4 + g) * 1024 + (l16 * 16 + 4 * i) * 4);
            u32x4 *dst = reinterpret_cast<u32x4 *>(tb + l16 * 128 + g * 32);
            dst[0] = u32x4{pack_bf16x2(t[0][0], t[0][1]), pack_bf16x2(t[0][2], t[0][3]), pack_bf16x2(t[1][0], t[1][1]),
                           pack_bf16x2(t[1][2], t[1][3])};
            dst[1] = u32x4{pack_bf16x2(t[2][0], t[2][1]), pack_bf16x2(t[2][2], t[2][3]), pack_bf16x2(t[3][0], t[3][1]),
                           pack_bf16x2(t[3][2], t[3][3])};
            u32x4 af[2][WNF];
            if (h == 0) {
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                    for (int f = 0; f < WNF; ++f) af[cc][f] = af0[cc][f];
            } else {
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                    for (int f = 0; f < WNF; ++f) {
                        const int ka = 64 * h + 32 * cc + 8 * g;
                        const unsigned row = row_of(f, l16);
                        af[cc][f] = bload16(ra, (row * (unsigned)a.lda + (unsigned)ka) * 2u +
                                                    (ka < a.lda && row != kNoRow ? 0u : kOOB));
                    }
            }
            // (this wave's own LDS writes above are what it reads here)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const u32x4 tf = *reinterpret_cast<const u32x4 *>(tb + l16 * 128 + (32 * cc + 8 * g) * 2);
#pragma unroll
                for (int f = 0; f < WNF; ++f) sum[f] = mfma16(af[cc][f], tf, sum[f]);
            }
        }
        if (h + 1 < a.r_pad / 64) {
            barrier_lds_sync();  // the next group's staging overwrites tst
            stage_t(h + 1);
        }
    }
    if (wave == 0) {
        if (a.glu) {
            const int n = 16 * c + 4 * g;
            if (l16 < a.M && n < a.F) {
                float o[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) o[v] = (sum[0][v] + bv[0][v]) * gelu_erf(sum[1][v] + bv[1][v]);
                store_out(a, l16, n, o);
            }
        } else {
#pragma unroll
            for (int f = 0; f < WNF; ++f) {
                const int n = n0 + 16 * f + 4 * g;
                if (l16 < a.M && n < a.N) {
                    const float o[4] = {sum[f][0] + bv[f][0], sum[f][1] + bv[f][1], sum[f][2] + bv[f][2],
                                        sum[f][3] + bv[f][3]};
                    store_out(a, l16, n, o);
                }
            }
        }
    }
}

template <int NQ>
hipError_t launch_fullk(const SArgs &a, int qf, hipStream_t s) {
    if (qf)
        hipLaunchKernelGGL((skinny_fullk_kernel<NQ, 1>), dim3(a.tiles_n), dim3(SNT), 0, s, a);
    else
        hipLaunchKernelGGL((skinny_fullk_kernel<NQ, 0>), dim3(a.tiles_n), dim3(SNT), 0, s, a);
    return hipGetLastError();
}

template <int MB, int NSTEPS>
hipError_t launch_sk(const SArgs &a, int qf, hipStream_t s) {
    if constexpr (x_lds_bytes<MB, NSTEPS>() + 4 * MB * 64 * 16 + 64 > LDS_MAX) {
        return hipErrorInvalidValue;
    } else {
        const int grid = a.tiles_n * a.splits;
        if (qf)
            hipLaunchKernelGGL((skinny_kernel<MB, NSTEPS, 1>), dim3(grid), dim3(SNT), 0, s, a);
        else
            hipLaunchKernelGGL((skinny_kernel<MB, NSTEPS, 0>), dim3(grid), dim3(SNT), 0, s, a);
        return hipGetLastError();
    }
}

template <int MB>
hipError_t launch_sk_steps(int k_slice, const SArgs &a, int qf, hipStream_t s) {
    switch (k_slice / 64) {
        case 8: return launch_sk<MB, 8>(a, qf, s);
        case 16: return launch_sk<MB, 16>(a, qf, s);
        case 32: return launch_sk<MB, 32>(a, qf, s);
        case 64: return launch_sk<MB, 64>(a, qf, s);
    }
    return hipErrorInvalidValue;
}

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

bool skinny_supports(int64_t M) { return M >= 1 && M <= SMAX_M; }

SkinnyPlan skinny_plan(int64_t M, int64_t K, int64_t N, int64_t r_pad, int64_t splits_hint, bool glu) {
    SkinnyPlan pl{};
    pl.mb = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    // Up to 16 rows, 2048 < K <= 8192 and enough 32-column work-groups to
    // fill most of the chip: all of K per work-group (no K slices).
    const int64_t groups32 = glu ? cdiv64(N / 2, 16) : cdiv64(N, 32);
    const int64_t nq = K <= 4096 ? 4 : 8;
    const int64_t pieces = (r_pad / 16) * nq;  // 16 ranks x one 256-element chunk of every wave's K quarter
    if (pl.mb == 1 && splits_hint <= 0 && K > 2048 && K <= 8192 && groups32 >= 192 && pieces <= groups32 &&
        pieces <= 256) {
        pl.fullk = 1;
        pl.nq = (int)nq;
        pl.tiles_n = (int)groups32;
        pl.k_slice = (int)K;
        pl.splits = 1;
        pl.groups = (int)(r_pad / 16);
        pl.t_kslice = 1024;
        pl.pps = (int)pieces;
        pl.pwg = pl.pps;
        pl.t_splits = (int)nq;
        pl.producers = r_pad > 0 ? pl.pps : 0;
        return pl;
    }
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

int64_t skinny_sync_words(const SkinnyPlan &pl) { return (int64_t)pl.tiles_n + 2; }

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
    if (p.glu && p.N % 2 != 0) return hipErrorInvalidValue;
    a.glu = p.glu;
    a.F = p.glu ? (int)(p.N / 2) : 0;
    a.N = p.glu ? pl.tiles_n * SBN : (int)p.N;  // the products' columns (partial sums' row length)
    a.NO = p.glu ? a.F : (int)p.N;
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
    a.fdone = p.sync + pl.tiles_n + 1;
    a.t_target = (unsigned)(pl.pps * pl.splits) + p.wait_extra;  // one bump per T piece
    a.wait_limit = p.wait_limit;
    a.err = p.err;
    if (p.r > 0 && (!p.err || p.wait_limit == 0)) return hipErrorInvalidValue;
    a.y_vec = (a.NO % 4 == 0) && ((uintptr_t)p.y % 16 == 0) && ((uintptr_t)p.partials % 16 == 0);
    a.out_f32 = p.out_f32;
    a.gelu = p.gelu;
    if (pl.fullk) {
        a.pwg = 0;  // (piece work-groups are the ids below pps)
        a.gen = p.gen;
        a.t_target = p.wait_extra;  // added to the count that completes this launch's pieces
        if (p.r > 0 && !p.gen) return hipErrorInvalidValue;
        return pl.nq == 4 ? launch_fullk<4>(a, p.q_format, s) : launch_fullk<8>(a, p.q_format, s);
    }
    switch (pl.mb) {
        case 1: return launch_sk_steps<1>(pl.k_slice, a, p.q_format, s);
        case 2: return launch_sk_steps<2>(pl.k_slice, a, p.q_format, s);
        case 4: return launch_sk_steps<4>(pl.k_slice, a, p.q_format, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ll
