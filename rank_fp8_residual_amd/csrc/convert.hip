// Decomposition side of LiteLinear on gfx950: the residual of a dense weight
// after its rank-r pair, quantised to e4m3fn with one per-tensor scale.
//
// The layer holds W ~ A B + s dec(Q) (LiteLinear README, page
// "moonmath-ai/LiteLinear", *Features*; LiteLinear.from_dense under *Usage*
// builds A and B by an SVD).  Given W and the pair, this file computes
//     R = W - A B                      (float32, never stored)
//     s = max |R| / 448  (1 when R is all zero)
//     Q = nearest e4m3fn to clamp(R / s, +-448), ties to even
// in two passes over W: in the first, each work-group writes max |R| over
// its tile to a slot of its own; in the second, each work-group first takes
// the maximum over all slots (a few KiB from L2), then recomputes R and
// writes the codes (and s).  No slot needs clearing between calls and no
// work-group waits for another, so one call is two launches.  A B runs on
// bf16 matrix cores (K = r); B's tile is transposed through LDS so that its
// fragments, like A's, hold 8 consecutive ranks per lane.
//
// quant_tensor_kernel does the same two passes for a float32 R given as is.
// The scale and the quotient R / s are correctly rounded float32 divisions
// (the quotients through a reciprocal and one exact correction, see
// Quotient), and the codes come from gfx950's scaled e4m3fn conversion at
// scale 1.
#include "device_common.hpp"
#include "launch.hpp"

namespace ll {
namespace {

typedef short i16x2 __attribute__((ext_vector_type(2)));

// 4 float32 -> 4 e4m3fn codes (lowest first), nearest with ties to even;
// |v| <= 448 by the caller's clamp.  The sources pass through an empty asm
// statement, as in the activation quantiser (the compiler has been seen to
// feed one source to several conversions).
__device__ __forceinline__ unsigned codes4(float a, float b, float c, float d) {
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
    i16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2{0, 0}, a, b, 1.0f, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, 1.0f, true);
    return __builtin_bit_cast(unsigned, w);
}

__device__ __forceinline__ float scale_from_amax(unsigned amax_bits) {
    const float amax = __builtin_bit_cast(float, amax_bits);
    return amax > 0.0f ? amax / 448.0f : 1.0f;
}

// The per-work-group maxima of the first pass (non-negative floats as bit
// patterns, which order like the floats): this thread's share, requested
// with 16-byte loads (slots past `parts` read as zero).  PER: loads per
// thread, enough for parts <= 4 * PER * threads.
template <int PER>
struct PartialMax {
    u32x4 v[PER];
    __device__ void request(const unsigned *part, int parts, int tid, int threads) {
        const rsrc_t r = make_rsrc(part, (int64_t)parts * 4);
#pragma unroll
        for (int i = 0; i < PER; ++i) v[i] = bload16(r, (unsigned)(tid + i * threads) * 16u);
    }
    __device__ unsigned thread_max() const {
        unsigned m = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = v[i][e] > m ? v[i][e] : m;
        return m;
    }
};

// Maximum of u over the work-group (every thread gets it); red holds one
// word per wave, and the call ends with the work-group's threads in step.
__device__ __forceinline__ unsigned wg_umax(unsigned u, unsigned *red, int nwaves) {
    u = wave_umax(u);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();  // red free (an earlier use is complete)
    if (lane == 0) red[wave] = u;
    __syncthreads();
    unsigned m = 0;
    for (int w = 0; w < nwaves; ++w) m = red[w] > m ? red[w] : m;
    return m;
}

__device__ __forceinline__ float clamp448(float q) { return q > 448.0f ? 448.0f : (q < -448.0f ? -448.0f : q); }

// R / s rounded to float32 (nearest, ties to even) exactly as the IEEE
// division gives it, for many R and one s.  FAST: in three FMA-unit
// operations instead of a full division each.  With y = 1/s correctly
// rounded (one true division), q = R y is within one ulp of R / s, the
// remainder R - s q is exact in one FMA, and q + (R - s q) y rounded once is
// the correctly rounded quotient (Markstein's theorem: P. Markstein,
// "Computation of elementary functions on the IBM RISC System/6000
// processor", IBM J. Res. Dev. 34(1), 1990).  The theorem needs a remainder
// free of underflow; for every quotient that can round to a nonzero e4m3fn
// code (|R / s| >= 2^-10) that holds when s >= 2^-60, so the fast form is
// only used for 2^-60 <= s <= 2^100 (quotient_fast); elsewhere each
// quotient is a true division.
template <bool FAST>
struct Quotient {
    float s, y;
    __device__ explicit Quotient(float s_) : s(s_), y(FAST ? 1.0f / s_ : 0.0f) {}
    __device__ __forceinline__ float operator()(float r) const {
        if constexpr (FAST) {
            const float q = r * y;
            return __builtin_fmaf(__builtin_fmaf(-q, s, r), y, q);
        } else {
            return r / s;
        }
    }
};
__device__ __forceinline__ bool quotient_fast(float s) { return s >= 0x1p-60f && s <= 0x1p100f; }

// First pass: max |v| over the work-group into its slot part[blockIdx.x].
__device__ __forceinline__ void wg_max_to_slot(float v, unsigned *part, unsigned *red, int nwaves) {
    const unsigned m = wg_umax(__builtin_bit_cast(unsigned, v), red, nwaves);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// ---------------------------------------------------------- float32 R as is

constexpr int QT_THREADS = 256;
constexpr int QT_MAX_GRID = 4096;  // both passes run this many work-groups at most

// Both passes run the same grid; part holds one slot per work-group.
template <bool QUANT>
__global__ void __launch_bounds__(QT_THREADS) quant_tensor_kernel(const float *__restrict__ R, int64_t n,
                                                                 unsigned char *__restrict__ codes, unsigned *part,
                                                                 float *scale_out) {
    __shared__ unsigned red[QT_THREADS / 64];
    const rsrc_t rr = make_rsrc(R, n * 4);
    const int64_t groups = (n + 3) / 4;
    float s = 1.0f, m = 0.0f;
    if constexpr (QUANT) {
        PartialMax<QT_MAX_GRID / (4 * QT_THREADS)> pm;
        pm.request(part, (int)gridDim.x, (int)threadIdx.x, QT_THREADS);
        s = scale_from_amax(wg_umax(pm.thread_max(), red, QT_THREADS / 64));
        if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
    }
    auto pass = [&](auto div) {
        for (int64_t gi = (int64_t)blockIdx.x * QT_THREADS + threadIdx.x; gi < groups;
             gi += (int64_t)gridDim.x * QT_THREADS) {
            const f32x4 v = __builtin_bit_cast(f32x4, bload16(rr, (unsigned)(gi * 16)));  // past n: zeros
            if (!QUANT) {
                m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
            } else {
                const unsigned c =
                    codes4(clamp448(div(v[0])), clamp448(div(v[1])), clamp448(div(v[2])), clamp448(div(v[3])));
                const int64_t i = gi * 4;
                if (i + 3 < n) {
                    *reinterpret_cast<unsigned *>(codes + i) = c;
                } else {
                    for (int e = 0; e < 4 && i + e < n; ++e) codes[i + e] = (unsigned char)(c >> (8 * e));
                }
            }
        }
    };
    if (QUANT && quotient_fast(s))
        pass(Quotient<QUANT>(s));  // one branch per work-group, no per-element test
    else
        pass(Quotient<false>(s));
    if (!QUANT) wg_max_to_slot(m, part, red, QT_THREADS / 64);
}

// ------------------------------------------------------- R = W - A B on MFMA

constexpr int RT = 128;        // output tile: RT rows of W x RT columns
constexpr int RK = 32;         // ranks per step
constexpr int R_THREADS = 256; // 4 waves, wave w owns rows 32 w .. 32 w + 31

struct RArgs {
    const unsigned char *W, *A, *B;
    unsigned char *codes;
    unsigned *part;  // one slot per tile (work-group)
    float *scale_out;
    int N, K, r;  // W is [N, K], A [N, r], B [r, K]
    int parts;    // tiles
};

constexpr int R_PART_PER = 4;  // slot loads per thread issued ahead (4096 slots; more are read in a loop)

template <bool QUANT>
__global__ void __launch_bounds__(R_THREADS) __attribute__((amdgpu_waves_per_eu(3))) residual_kernel(RArgs a) {
    // B's step tile transposed: bt[j][k], 32 ranks (64 bytes) per column,
    // rows padded by 16 bytes so the fragment reads spread over the banks;
    // two of them, for alternate steps.
    constexpr int BTS = RK * 2 + 16;
    // The W tile (rows of RT bf16) and then the tile's codes (rows of RT
    // bytes), both with rows padded by 16 bytes: memory sees whole row
    // segments in 16-byte lanes, the fragments read and write them through
    // LDS (the 16 rows of a fragment fall on distinct banks).
    constexpr int WS = RT * 2 + 16, CS = RT + 16;
    // bt is only used by the product loop and ws only after it, so they
    // share one array: 35 KiB per work-group, three work-groups per CU.
    constexpr int LDS_BYTES = 2 * RT * BTS > RT * WS ? 2 * RT * BTS : RT * WS;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    unsigned char *const bt = lds, *const ws = lds;
    __shared__ unsigned red[R_THREADS / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
    const int tiles_k = (a.K + RT - 1) / RT;
    const int n0 = (blockIdx.x / tiles_k) * RT, j0 = (blockIdx.x % tiles_k) * RT;
    const rsrc_t ra = make_rsrc(a.A, (int64_t)a.N * a.r * 2);
    const rsrc_t rb = make_rsrc(a.B, (int64_t)a.r * a.K * 2);
    const rsrc_t rw = make_rsrc(a.W, (int64_t)a.N * a.K * 2);
    // The second pass requests the first pass's slots before the tile: the
    // tile's loads queue behind them, and the wait for those covers them.
    PartialMax<R_PART_PER> pm;
    if constexpr (QUANT) pm.request(a.part, a.parts, tid, R_THREADS);

    // The W tile is requested first, 16 bytes per lane along rows (16 lanes
    // per 256-byte row segment, 16 rows per round), and lands while A B is
    // summed.  Rows past N and columns past K read as zero.
    constexpr int WROUNDS = RT * RT * 2 / (16 * R_THREADS);
    const int wrow = tid >> 4, wcol = 8 * (tid & 15);
    u32x4 wl[WROUNDS];
#pragma unroll
    for (int p = 0; p < WROUNDS; ++p) {
        const int n = n0 + 16 * p + wrow, j = j0 + wcol;
        const bool ok = n < a.N && j < a.K;  // K % 16 == 0: all eight columns or none
        wl[p] = bload16(rw, ((unsigned)n * (unsigned)a.K + (unsigned)j) * 2u + (ok ? 0u : kOOB));
    }

    // acc[fc][fr]: lane holds (A B)[n0 + 32 wave + 16 fr + l16][j0 + 16 fc + 4 g + v]
    f32x4 acc[RT / 16][2];
#pragma unroll
    for (int fc = 0; fc < RT / 16; ++fc)
#pragma unroll
        for (int fr = 0; fr < 2; ++fr) acc[fc][fr] = f32x4{0.f, 0.f, 0.f, 0.f};

    // B tile of a step: thread t loads ranks k0 + 4 (t / 32) .. +4 of columns
    // j0 + 4 (t % 32) .. +4 (four 8-byte loads, 256 contiguous bytes per rank
    // row across 32 lanes); A fragments: 16 bytes per row block.  The loads
    // of step k + 1 are in flight while step k is transposed and multiplied.
    const int kq = 4 * (tid >> 5), jq = 4 * (tid & 31), jb = j0 + jq;
    auto load_b = [&](int k0, u32x2 (&v)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = k0 + kq + e;
            v[e] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                           rb, ((unsigned)k * (unsigned)a.K + (unsigned)jb) * 2u + (k < a.r && jb < a.K ? 0u : kOOB),
                           0, 0));
        }
    };
    auto load_a = [&](int k0, u32x4 (&af)[2]) {
#pragma unroll
        for (int fr = 0; fr < 2; ++fr) {
            const int n = n0 + 32 * wave + 16 * fr + l16, k = k0 + 8 * g;
            af[fr] = bload16(ra, ((unsigned)n * (unsigned)a.r + (unsigned)k) * 2u + (n < a.N && k < a.r ? 0u : kOOB));
        }
    };
    // Two register sets, each refilled for the step two ahead as soon as its
    // contents are consumed (B's into LDS, A's into the products), so every
    // load has two steps of work to land behind.  (A copy from a set loaded
    // for the next step into the current one would wait for that load.)
    u32x2 bv0[4], bv1[4];
    u32x4 af0[2], af1[2];
    if (a.r > 0) {
        load_b(0, bv0);
        load_a(0, af0);
    }
    if (a.r > RK) {
        load_b(RK, bv1);
        load_a(RK, af1);
    }
    // This thread's maximum over its slots (the wait covers only them: they
    // were requested first); slots past those requested ahead, in a loop.
    unsigned pmax = 0;
    if constexpr (QUANT) {
        pmax = pm.thread_max();
        const rsrc_t rp = make_rsrc(a.part, (int64_t)a.parts * 4);
        for (int q = R_PART_PER * R_THREADS + tid; q < (a.parts + 3) / 4; q += R_THREADS) {
            const u32x4 v = bload16(rp, (unsigned)q * 16u);
#pragma unroll
            for (int e = 0; e < 4; ++e) pmax = v[e] > pmax ? v[e] : pmax;
        }
    }
    auto step = [&](int k0, int st, u32x2 (&bv)[4], u32x4 (&af)[2]) {
        // bt[st] was last read two steps ago, before the previous step's barrier.
        unsigned char *const b = bt + st * (RT * BTS);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // column jq + c: ranks kq .. kq + 3 = element c of each row load
            const unsigned lo = c & 1 ? (bv[0][c >> 1] >> 16) | (bv[1][c >> 1] & 0xFFFF0000u)
                                      : (bv[0][c >> 1] & 0xFFFFu) | (bv[1][c >> 1] << 16);
            const unsigned hi = c & 1 ? (bv[2][c >> 1] >> 16) | (bv[3][c >> 1] & 0xFFFF0000u)
                                      : (bv[2][c >> 1] & 0xFFFFu) | (bv[3][c >> 1] << 16);
            *reinterpret_cast<u32x2 *>(b + (jq + c) * BTS + kq * 2) = u32x2{lo, hi};
        }
        if (k0 + 2 * RK < a.r) load_b(k0 + 2 * RK, bv);
        __syncthreads();
#pragma unroll
        for (int fc = 0; fc < RT / 16; ++fc) {
            const u32x4 bf = *reinterpret_cast<const u32x4 *>(b + (16 * fc + l16) * BTS + 16 * g);
#pragma unroll
            for (int fr = 0; fr < 2; ++fr) acc[fc][fr] = mfma16(bf, af[fr], acc[fc][fr]);
        }
        if (k0 + 2 * RK < a.r) load_a(k0 + 2 * RK, af);
    };
    for (int k0 = 0; k0 < a.r; k0 += 2 * RK) {
        step(k0, 0, bv0, af0);
        if (k0 + RK < a.r) step(k0 + RK, 1, bv1, af1);
    }

    __syncthreads();  // the last step's bt reads are done before ws overwrites them
#pragma unroll
    for (int p = 0; p < WROUNDS; ++p) *reinterpret_cast<u32x4 *>(ws + (16 * p + wrow) * WS + 2 * wcol) = wl[p];
    __syncthreads();

    // R = W - A B for the lane's elements: row 32 wave + 16 fr + l16 of the
    // tile, columns 16 fc + 4 g .. + 3.
    const float s = QUANT ? scale_from_amax(wg_umax(pmax, red, R_THREADS / 64)) : 1.0f;
    float m = 0.0f;
    if (QUANT && blockIdx.x == 0 && tid == 0) *a.scale_out = s;
    unsigned cv[2][RT / 16];
    auto residual = [&](auto div) {
#pragma unroll
        for (int fr = 0; fr < 2; ++fr) {
            const int row = 32 * wave + 16 * fr + l16;
            const bool okn = n0 + row < a.N;
#pragma unroll
            for (int fc = 0; fc < RT / 16; ++fc) {
                const int col = 16 * fc + 4 * g;
                const bool ok = okn && j0 + col < a.K;
                const u32x2 w4 = *reinterpret_cast<const u32x2 *>(ws + row * WS + 2 * col);
                float rv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float w = bf16_to_f32((unsigned short)(w4[v >> 1] >> (16 * (v & 1))));
                    rv[v] = ok ? w - acc[fc][fr][v] : 0.0f;
                }
                if (!QUANT)
                    m = fmaxf(m, fmaxf(fmaxf(fabsf(rv[0]), fabsf(rv[1])), fmaxf(fabsf(rv[2]), fabsf(rv[3]))));
                else
                    cv[fr][fc] =
                        codes4(clamp448(div(rv[0])), clamp448(div(rv[1])), clamp448(div(rv[2])), clamp448(div(rv[3])));
            }
        }
    };
    if (QUANT && quotient_fast(s))
        residual(Quotient<QUANT>(s));  // one branch per work-group, no per-element test
    else
        residual(Quotient<false>(s));
    if (!QUANT) {
        wg_max_to_slot(m, a.part, red, R_THREADS / 64);
        return;
    }
    // Codes: into LDS in fragment order (over the W tile, once every wave
    // has read it), then out in whole 128-byte row segments.
    __syncthreads();
#pragma unroll
    for (int fr = 0; fr < 2; ++fr)
#pragma unroll
        for (int fc = 0; fc < RT / 16; ++fc)
            *reinterpret_cast<unsigned *>(ws + (32 * wave + 16 * fr + l16) * CS + 16 * fc + 4 * g) = cv[fr][fc];
    __syncthreads();
    constexpr int CROUNDS = RT * RT / (16 * R_THREADS);
    const int crow = tid >> 3, ccol = 16 * (tid & 7);
#pragma unroll
    for (int p = 0; p < CROUNDS; ++p) {
        const int row = 32 * p + crow, n = n0 + row, j = j0 + ccol;
        const u32x4 c = *reinterpret_cast<const u32x4 *>(ws + row * CS + ccol);
        if (n < a.N && j < a.K)  // K % 16 == 0: all sixteen codes or none
            *reinterpret_cast<u32x4 *>(a.codes + (int64_t)n * a.K + j) = c;
    }
}

}  // namespace

int64_t quant_tensor_slots(int64_t n) {
    const int64_t blocks = ((n + 3) / 4 + QT_THREADS - 1) / QT_THREADS;
    return blocks < 1 ? 1 : (blocks < QT_MAX_GRID ? blocks : QT_MAX_GRID);
}

int64_t residual_quant_slots(int64_t N, int64_t K) { return ((N + RT - 1) / RT) * ((K + RT - 1) / RT); }

hipError_t launch_quant_tensor(const float *R, int64_t n, void *codes, unsigned *part, float *scale_out,
                               hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (n * 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int grid = (int)quant_tensor_slots(n);
    hipLaunchKernelGGL(quant_tensor_kernel<false>, dim3(grid), dim3(QT_THREADS), 0, s, R, n,
                       (unsigned char *)codes, part, scale_out);
    hipLaunchKernelGGL(quant_tensor_kernel<true>, dim3(grid), dim3(QT_THREADS), 0, s, R, n,
                       (unsigned char *)codes, part, scale_out);
    return hipGetLastError();
}

hipError_t launch_residual_quant(const void *W, const void *A, const void *B, int64_t N, int64_t K, int64_t r,
                                 void *codes, unsigned *part, float *scale_out, hipStream_t s) {
    if (N <= 0 || K <= 0) return hipSuccess;
    const int64_t lim = (int64_t)1 << 31;
    if (N * K * 2 >= lim || N * r * 2 >= lim || r * K * 2 >= lim) return hipErrorInvalidValue;
    const int64_t tiles = residual_quant_slots(N, K);
    if (tiles >= lim / 4) return hipErrorInvalidValue;
    RArgs a{};
    a.W = (const unsigned char *)W;
    a.A = (const unsigned char *)A;
    a.B = (const unsigned char *)B;
    a.codes = (unsigned char *)codes;
    a.part = part;
    a.scale_out = scale_out;
    a.N = (int)N;
    a.K = (int)K;
    a.r = (int)r;
    a.parts = (int)tiles;
    hipLaunchKernelGGL(residual_kernel<false>, dim3((unsigned)tiles), dim3(R_THREADS), 0, s, a);
    hipLaunchKernelGGL(residual_kernel<true>, dim3((unsigned)tiles), dim3(R_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace ll
