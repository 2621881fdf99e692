// Skinny-M (HBM-bound) path of the fused LiteLinear forward on gfx950.
//
// The forward (LiteLinear README, page "moonmath-ai/LiteLinear", equation in
// the introduction):  y = (x B^T) A^T + scale * (x dec(Q)^T) + bias.
//
// With few rows the time is the time to stream Q (out * in bytes) from HBM
// once.  The reduction over `in` is split into slices so that enough
// work-groups run to keep every CU loading; the grid is
// (column tiles of 256 outputs) x (K slices).  A work-group:
//   * streams its 256 x k_slice block of Q codes with 128-bit buffer loads
//     straight into registers (16 codes per lane per fragment), D steps of 64
//     ahead, converts them exactly to bf16 and feeds
//     v_mfma_f32_16x16x32_bf16 against the x rows;
//   * computes its slice's share of T = x B^T on the same x registers
//     (T = sum over slices of T_slice, so (sum T_slice) A^T = sum T_slice A^T
//     and no separate pass over x is needed);
//   * forms scale * acc + T_slice A^T, with T_slice rounded once to bf16;
//   * writes that partial sum as float32 with device-coherent stores; the
//     last work-group of the column tile to finish (an atomic counter) reads
//     the slices back with device-coherent loads, adds them in slice order,
//     adds bias and stores y.  The result does not depend on which
//     work-group finishes last, and the counter is left at zero.
// With one slice the partial step is skipped and y is stored directly.
// Every load is a buffer load: reads past a descriptor's end return zero,
// so masking rows, columns and the K tail needs no branch.
#include "device_common.hpp"
#include "launch.hpp"

namespace ll {
namespace {

constexpr int SNT = 256;            // threads per work-group (4 waves)
constexpr int WNF = 4;              // 16-column fragments per wave
constexpr int SBN = 4 * WNF * 16;   // output columns per work-group
constexpr int SMAX_M = 64;          // largest M (4 row blocks of 16)

struct SArgs {
    const unsigned char *x, *B, *Q, *A, *bias;
    void *y;
    float *partials;
    unsigned *counters;
    float scale;
    int M, K, N, r, r_pad, lda, k_slice, splits;
    bool y_vec, out_f32;
};

// Operands of one 64-wide step of the reduction, as this lane holds them:
// lane l covers reduction elements [k + 16*(l/16), +16) of row (l % 16) of
// each 16-row fragment; both halves of 8 feed one matrix-core product each.
template <int MB, int RT>
struct Step {
    u32x4 q[WNF];              // 16 e4m3fn codes per Q fragment
    u32x4 x0[MB], x1[MB];      // 2 x 8 bf16 of x per row block
    u32x4 b0[RT], b1[RT];      // 2 x 8 bf16 of B per rank fragment
};

struct Bufs {
    rsrc_t q, x, b;
};

template <int MB, int RT>
__device__ __forceinline__ void load_step(Step<MB, RT> &st, const Bufs &bf, const SArgs &a, int k, int ke,
                                          int wave, int lane) {
    const int l16 = lane & 15;
    const int kl = k + 16 * (lane >> 4);
    // in % 16 == 0: a 16-element chunk is all in or all out.  Out-of-range
    // chunks get offset + kOOB (past every descriptor) rather than one shared
    // constant, so that no two loads become identical and get merged behind a
    // branch: every load stays an unconditional instruction.
    const unsigned oob = kl < ke ? 0u : kOOB;
#pragma unroll
    for (int f = 0; f < WNF; ++f) {
        const int row = wave * (WNF * 16) + f * 16 + l16;  // row within the column tile
        st.q[f] = bload16(bf.q, (unsigned)row * (unsigned)a.K + (unsigned)kl + oob);
    }
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        const unsigned off = ((unsigned)(b * 16 + l16) * (unsigned)a.K + (unsigned)kl) * 2u + oob;
        st.x0[b] = bload16(bf.x, off);
        st.x1[b] = bload16(bf.x, off + 16u);
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int rr = (wave + 4 * t) * 16 + l16;
        const unsigned off = ((unsigned)rr * (unsigned)a.K + (unsigned)kl) * 2u + oob;
        st.b0[t] = bload16(bf.b, off);
        st.b1[t] = bload16(bf.b, off + 16u);
    }
}

template <int MB, int RT>
__device__ __forceinline__ void compute_step(const Step<MB, RT> &st, f32x4 (&acc)[WNF][MB],
                                             f32x4 (&tacc)[RT][MB]) {
#pragma unroll
    for (int f = 0; f < WNF; ++f) {
        u32x4 h0, h1;
        fp8x16_to_bf16x16(st.q[f], h0, h1);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            acc[f][b] = mfma16(h0, st.x0[b], acc[f][b]);
            acc[f][b] = mfma16(h1, st.x1[b], acc[f][b]);
        }
    }
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            tacc[t][b] = mfma16(st.b0[t], st.x0[b], tacc[t][b]);
            tacc[t][b] = mfma16(st.b1[t], st.x1[b], tacc[t][b]);
        }
}

__device__ __forceinline__ void store_out(const SArgs &a, int m, int n, const float (&o)[4]) {
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

// Register stages of K steps in flight, from the per-step register cost
// (Q 16, x 8 per row block, B 8 per rank fragment): deep enough to keep
// ~32 KB per wave in flight, shallow enough not to spill.
template <int MB, int RT>
constexpr int skinny_depth() {
    constexpr int regs = 16 + 8 * MB + 8 * RT;
    constexpr int d = 200 / regs;
    return d > 6 ? 6 : (d < 2 ? 2 : d);
}

template <int MB, int RT, int NSTEPS>
__global__ void __launch_bounds__(SNT) skinny_kernel(SArgs a) {
    constexpr int DEPTH = skinny_depth<MB, RT>() < NSTEPS ? skinny_depth<MB, RT>() : NSTEPS;
    constexpr int TS_LD = RT * 64 + 8;  // bf16 per LDS row of the T slice (16-byte multiple)
    constexpr int KCH = RT * 2;         // 32-wide rank chunks of A per fragment
    __shared__ __attribute__((aligned(16))) unsigned short ts[MB * 16][TS_LD];
    __shared__ unsigned is_last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int tn = blockIdx.x, slice = blockIdx.y;
    const int n_tile = tn * SBN, nw = n_tile + wave * (WNF * 16);
    const int kb = slice * a.k_slice;
    const int ke = (kb + a.k_slice < a.K) ? kb + a.k_slice : a.K;
    const int rows_n = (a.N - n_tile) < SBN ? (a.N - n_tile) : SBN;

    Bufs bf;
    bf.q = make_rsrc(a.Q + (int64_t)n_tile * a.K, (int64_t)rows_n * a.K);
    bf.x = make_rsrc(a.x, (int64_t)a.M * a.K * 2);
    bf.b = make_rsrc(a.B, (int64_t)a.r * a.K * 2);
    // Built here, in uniform control flow, so that it stays in scalar
    // registers (inside divergent code every use would become a loop).
    const rsrc_t rp = make_rsrc(a.partials, (int64_t)a.splits * a.M * a.N * 4);

    // A fragments for the epilogue: for ranks up to 128 they are fetched now,
    // so their latency hides under the reduction (larger ranks load them per
    // chunk at the end).  Lane holds A[row][32 c + 8 g, +8) for chunk c.  A
    // rows are whole 16-byte chunks (lda % 8 == 0, zero padded past r); rows
    // past N read as zero.
    constexpr bool PREFETCH_A = RT <= 2;
    const rsrc_t ra = make_rsrc(a.A + (int64_t)n_tile * a.lda * 2, (int64_t)rows_n * a.lda * 2);
    auto load_a = [&](int f, int c) {
        const int row = wave * (WNF * 16) + f * 16 + l16, ka = 32 * c + 8 * g;
        return bload16(ra, ((unsigned)row * (unsigned)a.lda + (unsigned)ka) * 2u + (ka < a.lda ? 0u : kOOB));
    };
    u32x4 afr[WNF][PREFETCH_A ? KCH : 1];
    if constexpr (PREFETCH_A) {
#pragma unroll
        for (int f = 0; f < WNF; ++f)
#pragma unroll
            for (int c = 0; c < KCH; ++c) afr[f][c] = load_a(f, c);
    }

    f32x4 acc[WNF][MB], tacc[RT][MB];
#pragma unroll
    for (int f = 0; f < WNF; ++f)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int b = 0; b < MB; ++b) tacc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Reduction over this slice (NSTEPS steps of 64, fully unrolled) with a
    // ring of DEPTH register stages: the loads of step s + DEPTH - 1 are
    // issued before step s is computed, and scheduling barriers keep the
    // compiler from sinking them next to their uses.  Steps past the end of
    // `in` load zeros (out-of-range offsets) and add nothing.
    Step<MB, RT> st[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) load_step(st[d], bf, a, kb + 64 * d, ke, wave, lane);
#pragma unroll
    for (int s0 = 0; s0 < NSTEPS; ++s0) {
        if (s0 + DEPTH - 1 < NSTEPS)
            load_step(st[(s0 + DEPTH - 1) % DEPTH], bf, a, kb + 64 * (s0 + DEPTH - 1), ke, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
        compute_step(st[s0 % DEPTH], acc, tacc);
        __builtin_amdgcn_sched_barrier(0);
    }

    // T slice -> LDS as bf16: lane holds T[m = 16b + l16][16 rf + 4g + v].
    const int rfr = a.r_pad / 16;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int rf = wave + 4 * t;
        if (rf < rfr) {
#pragma unroll
            for (int b = 0; b < MB; ++b)
                *reinterpret_cast<u32x2 *>(&ts[b * 16 + l16][rf * 16 + 4 * g]) =
                    u32x2{pack_bf16x2(tacc[t][b][0], tacc[t][b][1]), pack_bf16x2(tacc[t][b][2], tacc[t][b][3])};
        }
    }
    __syncthreads();

#pragma unroll
    for (int f = 0; f < WNF; ++f)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[f][b] *= a.scale;

    // acc += T_slice A^T over the padded rank (A columns past r are zero).
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
        const int ka = 32 * c + 8 * g;
        if (32 * c >= a.r_pad) break;
        u32x4 bt[MB];
#pragma unroll
        for (int b = 0; b < MB; ++b) bt[b] = *reinterpret_cast<const u32x4 *>(&ts[b * 16 + l16][ka]);
#pragma unroll
        for (int f = 0; f < WNF; ++f) {
            const u32x4 av = PREFETCH_A ? afr[f][PREFETCH_A ? c : 0] : load_a(f, c);
#pragma unroll
            for (int b = 0; b < MB; ++b) acc[f][b] = mfma16(av, bt[b], acc[f][b]);
        }
    }

    // Lane holds acc[f][b][v] = y[m = 16b + l16][n = nw + 16f + 4g + v] (minus bias).
    if (a.splits > 1) {
        // Device-scope stores: visible to every XCD once they complete.
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
        // Every wave waits for its own stores to complete (device scope),
        // then the barrier; only then does the counter move.
        wait_vmcnt<0>();
        __syncthreads();
        if (tid == 0) is_last = bump_u32(&a.counters[tn]) == (unsigned)(a.splits - 1) ? 1u : 0u;
        __syncthreads();
        if (!is_last) return;
    }

    // Bias of this lane's columns, fetched before the partial sums so that
    // its latency overlaps theirs.
    const rsrc_t rb = make_rsrc(a.bias, a.bias ? (int64_t)a.N * 2 : 0);
    float bv[WNF][4];
#pragma unroll
    for (int f = 0; f < WNF; ++f) {
        const int n = nw + f * 16 + 4 * g;
#pragma unroll
        for (int v = 0; v < 4; ++v) bv[f][v] = bload_bf16(rb, (unsigned)(n + v));
    }

    if (a.splits > 1 && a.y_vec) {
        // Slices in batches of SB whose loads (every fragment of the lane)
        // are all in flight at once: one memory round trip per batch.  Each
        // element adds its slices in slice order, starting from zero, so the
        // sum does not depend on which work-group got here.  Out-of-range
        // slices, rows and columns read as zero.
        constexpr int SB = (32 / (WNF * MB)) > 0 ? 32 / (WNF * MB) : 1;
        const unsigned stride = (unsigned)a.M * (unsigned)a.N * 4u;
        f32x4 sum[WNF][MB];
#pragma unroll
        for (int f = 0; f < WNF; ++f)
#pragma unroll
            for (int b = 0; b < MB; ++b) sum[f][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < a.splits; s0 += SB) {
            f32x4 p[SB][WNF][MB];
#pragma unroll
            for (int u = 0; u < SB; ++u)
#pragma unroll
                for (int f = 0; f < WNF; ++f)
#pragma unroll
                    for (int b = 0; b < MB; ++b) {
                        const int n = nw + f * 16 + 4 * g, m = b * 16 + l16;
                        const bool ok = s0 + u < a.splits && m < a.M && n < a.N;
                        p[u][f][b] = bload16f_dc(rp, (unsigned)(s0 + u) * stride + (unsigned)(m * a.N + n) * 4u +
                                                         (ok ? 0u : kOOB));
                    }
#pragma unroll
            for (int u = 0; u < SB; ++u)
#pragma unroll
                for (int f = 0; f < WNF; ++f)
#pragma unroll
                    for (int b = 0; b < MB; ++b) sum[f][b] += p[u][f][b];
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
    if (a.splits > 1 && tid == 0) __hip_atomic_store(&a.counters[tn], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MB, int RT, int NSTEPS>
hipError_t launch_sk(const SArgs &a, int tiles_n, hipStream_t s) {
    hipLaunchKernelGGL((skinny_kernel<MB, RT, NSTEPS>), dim3(tiles_n, a.splits), dim3(SNT), 0, s, a);
    return hipGetLastError();
}

template <int MB, int RT>
hipError_t launch_sk_steps(const SArgs &a, int tiles_n, hipStream_t s) {
    switch (a.k_slice / 64) {
        case 4: return launch_sk<MB, RT, 4>(a, tiles_n, s);
        case 8: return launch_sk<MB, RT, 8>(a, tiles_n, s);
        case 16: return launch_sk<MB, RT, 16>(a, tiles_n, s);
    }
    return hipErrorInvalidValue;
}

// Row blocks (MB) x rank fragments per wave (RT) that are instantiated: the
// register budget allows RT <= 8 / MB (larger combinations would spill).
hipError_t launch_sk_m(const SArgs &a, int tiles_n, hipStream_t s) {
    const int rt = (a.r_pad + 63) / 64;
    if (a.M <= 16) {
        if (rt <= 1) return launch_sk_steps<1, 1>(a, tiles_n, s);
        if (rt <= 2) return launch_sk_steps<1, 2>(a, tiles_n, s);
        if (rt <= 4) return launch_sk_steps<1, 4>(a, tiles_n, s);
        if (rt <= 8) return launch_sk_steps<1, 8>(a, tiles_n, s);
    } else if (a.M <= 32) {
        if (rt <= 1) return launch_sk_steps<2, 1>(a, tiles_n, s);
        if (rt <= 2) return launch_sk_steps<2, 2>(a, tiles_n, s);
        if (rt <= 4) return launch_sk_steps<2, 4>(a, tiles_n, s);
    } else if (a.M <= SMAX_M) {
        if (rt <= 1) return launch_sk_steps<4, 1>(a, tiles_n, s);
        if (rt <= 2) return launch_sk_steps<4, 2>(a, tiles_n, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int skinny_col_tile() { return SBN; }

bool skinny_supports(int64_t M, int64_t r_pad) {
    const int64_t rt = (r_pad + 63) / 64;
    if (M <= 16) return rt <= 8;
    if (M <= 32) return rt <= 4;
    if (M <= SMAX_M) return rt <= 2;
    return false;
}

bool skinny_shape_ok(int64_t M, int64_t K, int64_t N, int64_t r_pad, int64_t splits) {
    // Every buffer descriptor must stay below 2^31 bytes.
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)SBN * K < lim && M * K * 2 < lim && r_pad * K * 2 < lim && (int64_t)SBN * r_pad * 2 < lim &&
           splits * M * N * 4 < lim && N * 2 < lim;
}

int skinny_slice_steps(int64_t K, int64_t N, int64_t splits_hint) {
    const int64_t tiles_n = (N + SBN - 1) / SBN;
    const int64_t ksteps = (K + 63) / 64;
    int64_t want = splits_hint > 0 ? splits_hint : (256 + tiles_n - 1) / tiles_n;  // ~one work-group per CU
    if (want < 1) want = 1;
    const int64_t per = (ksteps + want - 1) / want;
    return per <= 4 ? 4 : (per <= 8 ? 8 : 16);
}

hipError_t launch_skinny(const SkinnyProblem &p, const void *a_eff, hipStream_t s) {
    SArgs a{};
    a.x = (const unsigned char *)p.x;
    a.B = (const unsigned char *)p.B;
    a.Q = (const unsigned char *)p.Q;
    a.A = (const unsigned char *)a_eff;
    a.bias = (const unsigned char *)p.bias;
    a.y = p.y;
    a.partials = p.partials;
    a.counters = p.counters;
    a.scale = p.scale;
    a.M = (int)p.M;
    a.K = (int)p.K;
    a.N = (int)p.N;
    a.r = (int)p.r;
    a.r_pad = (int)p.r_pad;
    a.lda = a_eff == p.A ? (int)p.r : (int)p.r_pad;
    a.k_slice = (int)p.k_slice;
    a.splits = p.splits;
    a.y_vec = (p.N % 4 == 0) && ((uintptr_t)p.y % 16 == 0) && ((uintptr_t)p.partials % 16 == 0);
    a.out_f32 = p.out_f32;
    const int tiles_n = (int)((p.N + SBN - 1) / SBN);
    return launch_sk_m(a, tiles_n, s);
}

}  // namespace ll
