// Activations to e4m3fn for the fp8-activation mode of the fused LiteLinear
// forward on gfx950.
//
// The residual product y_res = scale * (x dec(Q)^T) (LiteLinear README, page
// "moonmath-ai/LiteLinear", equation in the introduction) can run on the fp8
// matrix cores when x is also held in e4m3fn (the README's fp8 residual is
// e4m3fn; the activation format and its scaling are this library's choice).
// Each row m gets one power-of-two scale 2^e: e is the smallest integer with
// max_j |x[m,j]| <= 448 * 2^e, at least -126 (-126 for an all-zero row), and
// code[m,j] is the e4m3fn value nearest to x[m,j] / 2^e, ties to the even
// code.  The division by 2^e is exact, so the rounding to e4m3fn is the only
// one.  A row holding a NaN or an infinity gets e = 0 and every code 0x7F.
//
// One wave per row: a first pass over the row finds max |x| (and any
// non-finite value), a second writes eight codes per lane per 16-byte group;
// rows of up to 8192 elements stay in registers between the two, longer
// ones are read again (from L2).  The scale comes from integer work on the
// bf16 bit patterns; the codes from gfx950's scaled e4m3fn conversion.
#include "device_common.hpp"
#include "launch.hpp"

namespace ll {
namespace {

constexpr int QWAVES = 4;  // rows (waves) per work-group

typedef short i16x2 __attribute__((ext_vector_type(2)));

// Codes of one 16-byte group (8 bf16, lowest first) given the row's scale
// 2^e.  gfx950's scaled conversion divides by the scale (exact for a power of
// two) and rounds to the nearest e4m3fn value, ties to even, keeping the sign
// of zero; its result is only checked against the pages' format by the tests
// (bit for bit against an independent quantiser, every bf16 value).  A row
// holding a NaN or an infinity gets 0x7F throughout.
__device__ __forceinline__ u32x2 codes8(u32x4 v, float scale, bool bad) {
    // The four source dwords pass through an empty asm statement: without
    // it the compiler has been seen to feed the first dword to all four
    // conversions.
    unsigned w0 = v.x, w1 = v.y, w2 = v.z, w3 = v.w;
    asm volatile("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
    i16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(i16x2{0, 0}, __builtin_bit_cast(bf16x2, w0), scale, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2, w1), scale, true);
    i16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(i16x2{0, 0}, __builtin_bit_cast(bf16x2, w2), scale, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(bf16x2, w3), scale, true);
    const u32x2 c = u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    return bad ? u32x2{0x7F7F7F7Fu, 0x7F7F7F7Fu} : c;
}

// NCH > 0: the row (at most NCH x 512 elements) is read once into registers,
// all loads in flight together.  NCH == 0: any length, read twice (the
// second pass from L2).
template <int NCH>
__global__ void __launch_bounds__(QWAVES * 64) quant_rows_kernel(const unsigned short *__restrict__ x,
                                                                unsigned char *__restrict__ codes,
                                                                float *__restrict__ scales, int M, int K,
                                                                int64_t ldx) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * QWAVES + (threadIdx.x >> 6);
    if (m >= M) return;
    const rsrc_t rx = make_rsrc(x + (int64_t)m * ldx, (int64_t)K * 2);
    // Pass 1: max |x| as bit patterns (|bf16| orders like its bits) and a
    // flag for exponent field 0xFF (infinity or NaN); past K reads zero.
    unsigned amax = 0, bad = 0;
    auto scan = [&](const u32x4 &v) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const unsigned h = (v[w] >> (16 * hh)) & 0x7FFFu;
                amax = h > amax ? h : amax;
                bad |= (h >= 0x7F80u) ? 1u : 0u;
            }
        }
    };
    auto load = [&](int k) { return bload16(rx, (unsigned)k * 2u + (k < K ? 0u : kOOB)); };
    u32x4 row[NCH > 0 ? NCH : 1];
    if constexpr (NCH > 0) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) row[c] = load(512 * c + 8 * lane);
#pragma unroll
        for (int c = 0; c < NCH; ++c) scan(row[c]);
    } else {
        for (int k0 = 0; k0 < K; k0 += 512) scan(load(k0 + 8 * lane));
    }
    // one wave maximum of (bad, amax): bit 16 set if any lane saw a
    // non-finite value, and then the row gets e = 0 whatever amax is
    {
        const unsigned key = wave_umax((bad << 16) | amax);
        bad = key >> 16;
        amax = key & 0xFFFFu;
    }
    // Scale exponent: amax = mant 2^ex with mant in [0.5, 1); 448 2^e is
    // 0.875 2^(e + 9).  A bf16 pattern below 0x0080 (subnormal) is under
    // 2^-126, and so is its e before the clamp.
    int e = -126;
    if (bad) {
        e = 0;
    } else if (amax >= 0x0080u) {
        const int ex = (int)(amax >> 7) - 126;      // float exponent of frexp
        const bool over = (amax & 0x7Fu) > 0x60u;  // mantissa of amax above 1.75
        e = over ? ex - 8 : ex - 9;
        e = e < -126 ? -126 : e;
    }
    const float scale = __builtin_ldexpf(1.0f, e);
    if (lane == 0) scales[m] = scale;
    // Pass 2: codes, eight per lane per 16-byte group.
    unsigned char *crow = codes + (int64_t)m * K;
    if constexpr (NCH > 0) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int k = 512 * c + 8 * lane;
            if (k < K) *reinterpret_cast<u32x2 *>(crow + k) = codes8(row[c], scale, bad != 0);
        }
    } else {
        for (int k0 = 0; k0 < K; k0 += 512) {
            const int k = k0 + 8 * lane;
            if (k >= K) break;
            *reinterpret_cast<u32x2 *>(crow + k) = codes8(load(k), scale, bad != 0);
        }
    }
}

}  // namespace

hipError_t launch_quant_rows(const void *x, int64_t ldx, void *codes, float *scales, int64_t M, int64_t K,
                             hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (K % 8 != 0 || ldx % 8 != 0 || ldx < K || K * 2 >= ((int64_t)1 << 31) || M >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    const int grid = (int)((M + QWAVES - 1) / QWAVES);
    const int nch = (int)((K + 511) / 512);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(grid), dim3(QWAVES * 64), 0, s, (const unsigned short *)x,
                           (unsigned char *)codes, scales, (int)M, (int)K, ldx);
    };
    if (nch <= 1)
        go(quant_rows_kernel<1>);
    else if (nch <= 2)
        go(quant_rows_kernel<2>);
    else if (nch <= 4)
        go(quant_rows_kernel<4>);
    else if (nch <= 8)
        go(quant_rows_kernel<8>);
    else if (nch <= 16)
        go(quant_rows_kernel<16>);
    else
        go(quant_rows_kernel<0>);
    return hipGetLastError();
}

}  // namespace ll
