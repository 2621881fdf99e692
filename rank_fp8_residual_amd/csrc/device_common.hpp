// Device helpers shared by the gfx950 kernels of the fused LiteLinear forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ll {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// 16x16x32 bf16 matrix-core product, float32 accumulate: c += a * b^T where
// lane l holds row (l % 16) of `a` and of `b`, and 8 of the 32 reduction
// indices (the same 8 for both operands).  The result tile D[i][j], i indexing
// a's rows and j b's rows, sits in lane l as D[4*(l/16) + v][l % 16], v = 0..3.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Four e4m3fn codes (bytes of `w`, lowest first) -> four bf16 values (two
// dwords, lowest first).  gfx950's conversion instruction reads the OCP
// e4m3fn encoding; with a multiplier of exactly 1.0 it is exact, because
// every e4m3fn value (subnormals included) is a bf16 value.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(unsigned w) {
    bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// 16 e4m3fn codes -> 16 bf16 (two 8-element halves).
__device__ __forceinline__ void fp8x16_to_bf16x16(u32x4 q, u32x4 &h0, u32x4 &h1) {
    u32x2 a = fp8x4_to_bf16x4(q.x), b = fp8x4_to_bf16x4(q.y);
    u32x2 c = fp8x4_to_bf16x4(q.z), d = fp8x4_to_bf16x4(q.w);
    h0 = u32x4{a.x, a.y, b.x, b.y};
    h1 = u32x4{c.x, c.y, d.x, d.y};
}

// float32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
    unsigned u = __builtin_bit_cast(unsigned, f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu))
        return (unsigned short)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (unsigned short)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
    return __builtin_bit_cast(float, (unsigned)h << 16);
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    return (unsigned)f32_to_bf16_rne(a) | ((unsigned)f32_to_bf16_rne(b) << 16);
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

}  // namespace ll
