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

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 16x16x128 e4m3fn matrix-core product, float32 accumulate: c += a * b^T with
// both operands e4m3fn codes.  Lane l holds row (l % 16) of `a` and of `b`
// and 32 of the 128 reduction indices, the same 32 for both operands (a0/b0
// the first 16 bytes, a1/b1 the next 16); the result layout is mfma16's.
// Every product of two e4m3fn values is exact in float32.  The instruction's
// block scales are left at 2^0 (E8M0 code 127).
__device__ __forceinline__ f32x4 mfma16_f8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x4 c) {
    const i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
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

// e4m3fnuz, the residual's format on AMD hardware (LiteLinear README,
// Features): exponent bias 8 instead of 7, no negative zero, no infinities.
// Every code but three decodes to exactly half its e4m3fn value, so the
// e4m3fn conversion at a multiplier of 0.5 is exact for them.  The three
// exceptions: 0x7F and 0xFF (e4m3fn NaN, e4m3fnuz +-240) and 0x80 (e4m3fn
// -0, e4m3fnuz NaN).  A per-tensor quantiser emits +-240 only where it hits
// the tensor's largest magnitude, so the fix-up below is rare; callers test
// for it first with fnuz_special_or().
__device__ __forceinline__ unsigned fnuz_special_or(unsigned acc, unsigned w) {
    // Byte-wise, with no carry between bytes (t's bytes are at most 0x7F):
    // t + 0x01 has bit 7 set exactly for the bytes 0x7F and 0xFF, and
    // ~(t + 0x7F) has bit 7 set exactly for the bytes whose low 7 bits are
    // zero, of which w's sign bit keeps 0x80.  Only bits 7 of each byte
    // (mask 0x80808080) of the result mean anything.
    const unsigned t = w & 0x7F7F7F7Fu;
    return acc | (t + 0x01010101u) | (~(t + 0x7F7F7F7Fu) & w);
}
__device__ __forceinline__ bool fnuz_any_special(unsigned acc) { return (acc & 0x80808080u) != 0u; }

// The three exceptional e4m3fnuz codes of `w`, patched into the bf16 pairs
// that the halving conversion produced for it: 0x7F -> 240 (bf16 0x4370),
// 0xFF -> -240 (0xC370), 0x80 -> NaN (0x7FC0).
__device__ __forceinline__ u32x2 fnuz_patch(unsigned w, u32x2 r) {
    unsigned v[2] = {r.x, r.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned b = (w >> (8 * i)) & 0xFFu;
        const unsigned h = b == 0x7Fu ? 0x4370u : (b == 0xFFu ? 0xC370u : 0x7FC0u);
        const unsigned m = 0xFFFFu << (16 * (i & 1));
        if (b == 0x7Fu || b == 0xFFu || b == 0x80u) v[i >> 1] = (v[i >> 1] & ~m) | ((h << (16 * (i & 1))) & m);
    }
    return u32x2{v[0], v[1]};
}

// The exceptional e4m3fnuz codes of `w` alone, as bf16 pairs (the layout
// of the halving conversion's result; every other code gives 0), and `w`
// with those codes replaced by 0x00 (zero).  The product of the two parts
// adds up to the product of the exact decode.
__device__ __forceinline__ u32x2 fnuz_special_values(unsigned w) {
    unsigned v[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned b = (w >> (8 * i)) & 0xFFu;
        const unsigned h = b == 0x7Fu ? 0x4370u : (b == 0xFFu ? 0xC370u : (b == 0x80u ? 0x7FC0u : 0u));
        v[i >> 1] |= h << (16 * (i & 1));
    }
    return u32x2{v[0], v[1]};
}
__device__ __forceinline__ unsigned fnuz_without_specials(unsigned w) {
    unsigned r = w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned b = (w >> (8 * i)) & 0xFFu;
        if (b == 0x7Fu || b == 0xFFu || b == 0x80u) r &= ~(0xFFu << (8 * i));
    }
    return r;
}

// Four residual codes -> four bf16 values: QF = 0 e4m3fn, QF = 1 e4m3fnuz
// (halving conversion; PATCH = true also fixes the three exceptional codes).
template <int QF, bool PATCH = false>
__device__ __forceinline__ u32x2 q8x4_to_bf16x4(unsigned w) {
    if constexpr (QF == 0) {
        return fp8x4_to_bf16x4(w);
    } else {
        const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 0.5f, false);
        const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 0.5f, true);
        const u32x2 r{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
        return PATCH ? fnuz_patch(w, r) : r;
    }
}

// Maximum of u over the wave (every lane gets it): within each row of 16
// lanes a running maximum from lanes 1, 2, 4, 8 below (DPP row shifts,
// lanes without a source keep their value), which leaves each row's maximum
// in its lane 15, then the four rows' lanes 15 combined as scalars.
__device__ __forceinline__ unsigned wave_umax(unsigned u) {
    auto up = [](unsigned a, unsigned b) { return a > b ? a : b; };
    u = up(u, (unsigned)__builtin_amdgcn_update_dpp((int)u, (int)u, 0x111, 0xF, 0xF, false));  // row_shr:1
    u = up(u, (unsigned)__builtin_amdgcn_update_dpp((int)u, (int)u, 0x112, 0xF, 0xF, false));  // row_shr:2
    u = up(u, (unsigned)__builtin_amdgcn_update_dpp((int)u, (int)u, 0x114, 0xF, 0xF, false));  // row_shr:4
    u = up(u, (unsigned)__builtin_amdgcn_update_dpp((int)u, (int)u, 0x118, 0xF, 0xF, false));  // row_shr:8
    const unsigned r0 = (unsigned)__builtin_amdgcn_readlane((int)u, 15), r1 = (unsigned)__builtin_amdgcn_readlane((int)u, 31);
    const unsigned r2 = (unsigned)__builtin_amdgcn_readlane((int)u, 47), r3 = (unsigned)__builtin_amdgcn_readlane((int)u, 63);
    return up(up(r0, r1), up(r2, r3));
}

// True on every lane when `p` holds on any lane of the wave.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// The exact GELU, v Phi(v) = 0.5 v (1 + erf(v / sqrt(2))) (Hendrycks and
// Gimpel, 2016), with the device library's erff: the gate's activation of
// the gated epilogue (GEGLU).
__device__ __forceinline__ float gelu_erf(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

// GELU in its tanh approximation (Hendrycks and Gimpel, "Gaussian Error
// Linear Units (GELUs)", 2016): 0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v +
// 0.044715 v^3).  Since 0.5 (1 + tanh(u)) = 1 / (1 + e^(-2u)), it is
// computed as v / (1 + 2^(-2u log2 e)) with the hardware's exp2 and
// reciprocal (about 1 ulp each): no cancellation near 0, and -0 or v in the
// tails.
__device__ __forceinline__ float gelu_tanh(float v) {
    const float u = 0.7978845608028654f * (v + 0.044715f * v * v * v);
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.8853900817779268f * u));
}

// float32 -> bf16 bits, round to nearest even: gfx950's conversion
// instruction (v_cvt_pk_bf16_f32) under the default rounding mode.
__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(unsigned short, (__bf16)f);
}

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
    return __builtin_bit_cast(float, (unsigned)h << 16);
}

// Two floats -> two bf16 (round to nearest even) in one dword, a low.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(unsigned, v);
}

// ---- buffer (descriptor-based) loads: an offset at or past the descriptor's
// byte count reads as zero, so masking needs no branch.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Added to an offset to push it past every descriptor built here (all are
// below 2^31 bytes, so real offset + kOOB is still out of range).
constexpr unsigned kOOB = 0x80000000u;

// Raw buffer over [base, base + bytes); bytes must stay below 2^31.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// Only whole 16-byte results are used from these loads: extracting single
// elements of a buffer-load result has been seen to shrink the load wrongly.
__device__ __forceinline__ u32x4 bload16(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One bf16 element of a row (element index n, row held by r with 2 bytes per
// element) as a float; past the row's end, or with an empty descriptor, it
// reads as zero.  There is no branch, so a run of these loads stays in
// flight together and costs one memory round trip.
__device__ __forceinline__ float bload_bf16(rsrc_t r, unsigned n) {
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, n * 2u, 0, 0));
}

// Cache policy of a load or store.  kDeviceCoherent (the sc1 bit) makes a
// load read, and a store write, at device scope: it never returns a line
// that another XCD's L2 has made stale, and a store is complete (vmcnt)
// only once it is visible to every XCD.  Data handed between work-groups of
// one launch travels this way, so no fence has to write back or invalidate
// a whole L2.
constexpr int kCached = 0;
constexpr int kDeviceCoherent = 16;
// Streamed once (the nt bit): the lines are not kept for reuse, which leaves
// the caches to data that is read again.
constexpr int kNonTemporal = 2;

// bload16 for data read exactly once (kNonTemporal).
__device__ __forceinline__ u32x4 bload16_nt(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
}

// 16 bytes per lane from the buffer straight into LDS: lane l's bytes land at
// lds + 16 * l (lds is wave-uniform).  Counts against vmcnt like any load.
template <int POLICY = kCached>
__device__ __forceinline__ void bload16_lds(rsrc_t r, void *lds, unsigned off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, off, 0, 0, POLICY);
}

// 16-byte device-coherent load, returned as a whole float vector: callers
// only combine it as a vector (see bload16 on element extraction).
__device__ __forceinline__ f32x4 bload16f_dc(rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceCoherent));
}

template <int POLICY>
__device__ __forceinline__ void bstore16(rsrc_t r, unsigned off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, POLICY);
}

template <int POLICY>
__device__ __forceinline__ void bstore8(rsrc_t r, unsigned off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, POLICY);
}

// Device-scope counter read without acquire side effects (no cache
// invalidation), for polling.
__device__ __forceinline__ unsigned poll_u32(const unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned bump_u32(unsigned *p) {
    return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A bounded wait for other work-groups of the launch gave up: set the
// handle's error word (host memory mapped into the device, written at system
// scope), which the host turns into a status.  The kernel then carries on,
// so it still ends normally; its output is undefined.
__device__ __forceinline__ void report_wait_timeout(unsigned *err) {
    __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, others left open).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// A compile-time integer, and a loop over B .. E - 1 that calls f(CInt<i>{})
// for each i: the loop is always unrolled, whatever the size of its body,
// so that the body can use i as a constant (template arguments, register
// array indices).
template <int I>
struct CInt {
    static constexpr int value = I;
};
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(CInt<B>{});
        static_for<B + 1, E>(f);
    }
}

// Work-group barrier without a memory fence (loads may stay in flight).
__device__ __forceinline__ void barrier_nofence() { __builtin_amdgcn_s_barrier(); }

// The same barrier, also a compiler barrier for memory accesses: LDS reads
// written after it are not moved above it (the s_barrier intrinsic alone
// orders no memory access), and no wait for loads in flight is added (a
// fence would wait for every load that writes LDS).
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Waits until this wave's LDS reads and writes have completed.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Work-group barrier that the instruction scheduler moves nothing across
// (neither memory accesses nor arithmetic), for code whose phases between
// barriers are chosen on purpose.
__device__ __forceinline__ void pp_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// barrier_lds after this wave's own LDS reads and writes have completed
// (lgkmcnt 0): LDS written before it by any wave is what reads after it see.
__device__ __forceinline__ void barrier_lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left open
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace ll
