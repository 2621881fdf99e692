// Decomposition side of LiteLinear on gfx950: the residual of a dense weight
// after its rank-r pair, quantised to e4m3fn with one per-tensor scale.
//
// The layer holds W ~ A B + s dec(Q) (LiteLinear README, page
// "moonmath-ai/LiteLinear", *Features*; LiteLinear.from_dense under *Usage*
// builds A and B by an SVD).  Given W and the pair, this file computes
//     R = W - A B                      (float32, never stored)
//     s = max |R| / 448  (1 when R is all zero)
//     Q = nearest e4m3fn to clamp(R / s, +-448), ties to even
// in two passes over W: the first reduces max |R| into one device word, the
// second recomputes R and writes the codes (and s).  A B runs on bf16 matrix
// cores (K = r); B's tile is transposed through LDS so that its fragments,
// like A's, hold 8 consecutive ranks per lane.
//
// quant_tensor_kernel does the same two passes for a float32 R given as is.
// The scale and the quotient R / s are correctly rounded float32 divisions,
// and the codes come from gfx950's scaled e4m3fn conversion at scale 1.
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

__device__ __forceinline__ float scale_of(const unsigned *amax_bits) {
    const float amax = __builtin_bit_cast(float, *amax_bits);
    return amax > 0.0f ? amax / 448.0f : 1.0f;
}

__device__ __forceinline__ float clamp448(float q) { return q > 448.0f ? 448.0f : (q < -448.0f ? -448.0f : q); }

// max |v| over a work-group into *amax_bits (non-negative floats order like
// their bit patterns, so an unsigned atomic max is exact and order-free).
__device__ __forceinline__ void wg_max(float v, unsigned *amax_bits, unsigned *red, int nwaves) {
    unsigned u = __builtin_bit_cast(unsigned, v);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const unsigned o = __shfl_xor(u, off);
        u = o > u ? o : u;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = u;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned m = 0;
        for (int w = 0; w < nwaves; ++w) m = red[w] > m ? red[w] : m;
        if (m) __hip_atomic_fetch_max(amax_bits, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------- float32 R as is

constexpr int QT_THREADS = 256;

template <bool QUANT>
__global__ void __launch_bounds__(QT_THREADS) quant_tensor_kernel(const float *__restrict__ R, int64_t n,
                                                                 unsigned char *__restrict__ codes,
                                                                 unsigned *amax_bits, float *scale_out) {
    __shared__ unsigned red[QT_THREADS / 64];
    const rsrc_t rr = make_rsrc(R, n * 4);
    const int64_t groups = (n + 3) / 4;
    float s = 1.0f, m = 0.0f;
    if (QUANT) {
        s = scale_of(amax_bits);
        if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
    }
    for (int64_t gi = (int64_t)blockIdx.x * QT_THREADS + threadIdx.x; gi < groups;
         gi += (int64_t)gridDim.x * QT_THREADS) {
        const f32x4 v = __builtin_bit_cast(f32x4, bload16(rr, (unsigned)(gi * 16)));  // past n: zeros
        if (!QUANT) {
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
        } else {
            const unsigned c = codes4(clamp448(v[0] / s), clamp448(v[1] / s), clamp448(v[2] / s), clamp448(v[3] / s));
            const int64_t i = gi * 4;
            if (i + 3 < n) {
                *reinterpret_cast<unsigned *>(codes + i) = c;
            } else {
                for (int e = 0; e < 4 && i + e < n; ++e) codes[i + e] = (unsigned char)(c >> (8 * e));
            }
        }
    }
    if (!QUANT) wg_max(m, amax_bits, red, QT_THREADS / 64);
}

// ------------------------------------------------------- R = W - A B on MFMA

constexpr int RT = 128;        // output tile: RT rows of W x RT columns
constexpr int RK = 32;         // ranks per step
constexpr int R_THREADS = 256; // 4 waves, wave w owns rows 32 w .. 32 w + 31

struct RArgs {
    const unsigned char *W, *A, *B;
    unsigned char *codes;
    unsigned *amax_bits;
    float *scale_out;
    int N, K, r;  // W is [N, K], A [N, r], B [r, K]
};

template <bool QUANT>
__global__ void __launch_bounds__(R_THREADS) residual_kernel(RArgs a) {
    // B's step tile transposed: bt[j][k], 32 ranks (64 bytes) per column,
    // rows padded by 16 bytes so the fragment reads spread over the banks;
    // two of them, for alternate steps.
    constexpr int BTS = RK * 2 + 16;
    __shared__ __attribute__((aligned(16))) unsigned char bt[2 * RT * BTS];
    // The W tile (rows of RT bf16) and then the tile's codes (rows of RT
    // bytes), both with rows padded by 16 bytes: memory sees whole row
    // segments in 16-byte lanes, the fragments read and write them through
    // LDS (the 16 rows of a fragment fall on distinct banks).
    constexpr int WS = RT * 2 + 16, CS = RT + 16;
    __shared__ __attribute__((aligned(16))) unsigned char ws[RT * WS];
    __shared__ unsigned red[R_THREADS / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
    const int tiles_k = (a.K + RT - 1) / RT;
    const int n0 = (blockIdx.x / tiles_k) * RT, j0 = (blockIdx.x % tiles_k) * RT;
    const rsrc_t ra = make_rsrc(a.A, (int64_t)a.N * a.r * 2);
    const rsrc_t rb = make_rsrc(a.B, (int64_t)a.r * a.K * 2);
    const rsrc_t rw = make_rsrc(a.W, (int64_t)a.N * a.K * 2);

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
    u32x2 bv[4], bn[4];
    u32x4 af[2], an[2];
    if (a.r > 0) {
        load_b(0, bv);
        load_a(0, af);
    }
    for (int k0 = 0, st = 0; k0 < a.r; k0 += RK, st ^= 1) {
        if (k0 + RK < a.r) {
            load_b(k0 + RK, bn);
            load_a(k0 + RK, an);
        }
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
        __syncthreads();
#pragma unroll
        for (int fc = 0; fc < RT / 16; ++fc) {
            const u32x4 bf = *reinterpret_cast<const u32x4 *>(b + (16 * fc + l16) * BTS + 16 * g);
#pragma unroll
            for (int fr = 0; fr < 2; ++fr) acc[fc][fr] = mfma16(bf, af[fr], acc[fc][fr]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = bn[e];
        af[0] = an[0];
        af[1] = an[1];
    }

#pragma unroll
    for (int p = 0; p < WROUNDS; ++p) *reinterpret_cast<u32x4 *>(ws + (16 * p + wrow) * WS + 2 * wcol) = wl[p];
    __syncthreads();

    // R = W - A B for the lane's elements: row 32 wave + 16 fr + l16 of the
    // tile, columns 16 fc + 4 g .. + 3.
    float s = 1.0f, m = 0.0f;
    if (QUANT) {
        s = scale_of(a.amax_bits);
        if (blockIdx.x == 0 && tid == 0) *a.scale_out = s;
    }
    unsigned cv[2][RT / 16];
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
                cv[fr][fc] = codes4(clamp448(rv[0] / s), clamp448(rv[1] / s), clamp448(rv[2] / s), clamp448(rv[3] / s));
        }
    }
    if (!QUANT) {
        wg_max(m, a.amax_bits, red, R_THREADS / 64);
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

hipError_t launch_quant_tensor(const float *R, int64_t n, void *codes, unsigned *amax_bits, float *scale_out,
                               hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (n * 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int64_t groups = (n + 3) / 4;
    const int grid = (int)((groups + QT_THREADS - 1) / QT_THREADS < 4096 ? (groups + QT_THREADS - 1) / QT_THREADS : 4096);
    hipError_t e = hipMemsetAsync(amax_bits, 0, sizeof(unsigned), s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(quant_tensor_kernel<false>, dim3(grid), dim3(QT_THREADS), 0, s, R, n,
                       (unsigned char *)codes, amax_bits, scale_out);
    hipLaunchKernelGGL(quant_tensor_kernel<true>, dim3(grid), dim3(QT_THREADS), 0, s, R, n,
                       (unsigned char *)codes, amax_bits, scale_out);
    return hipGetLastError();
}

hipError_t launch_residual_quant(const void *W, const void *A, const void *B, int64_t N, int64_t K, int64_t r,
                                 void *codes, unsigned *amax_bits, float *scale_out, hipStream_t s) {
    if (N <= 0 || K <= 0) return hipSuccess;
    const int64_t lim = (int64_t)1 << 31;
    if (N * K * 2 >= lim || N * r * 2 >= lim || r * K * 2 >= lim) return hipErrorInvalidValue;
    RArgs a{};
    a.W = (const unsigned char *)W;
    a.A = (const unsigned char *)A;
    a.B = (const unsigned char *)B;
    a.codes = (unsigned char *)codes;
    a.amax_bits = amax_bits;
    a.scale_out = scale_out;
    a.N = (int)N;
    a.K = (int)K;
    a.r = (int)r;
    const int64_t tiles = ((N + RT - 1) / RT) * ((K + RT - 1) / RT);
    if (tiles >= lim) return hipErrorInvalidValue;
    hipError_t e = hipMemsetAsync(amax_bits, 0, sizeof(unsigned), s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(residual_kernel<false>, dim3((unsigned)tiles), dim3(R_THREADS), 0, s, a);
    hipLaunchKernelGGL(residual_kernel<true>, dim3((unsigned)tiles), dim3(R_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace ll
