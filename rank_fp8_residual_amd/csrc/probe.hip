// HBM read ceiling probe: streams a device buffer once, as the skinny path
// streams its residual codes, so that a measured rate has the chip's own
// plain-read rate beside it (not part of the forward).
//
// Each work-group reads one contiguous span of the buffer; every load
// instruction moves 1 KiB per wave (16 bytes per lane, coalesced), UNROLL of
// them in flight per lane.  The loaded words are folded by XOR into one word
// per work-group, stored to `sink` so that nothing is optimised away.
#include "device_common.hpp"
#include "launch.hpp"

namespace ll {
namespace {

constexpr int PNT = 256;  // threads per work-group

template <int UNROLL, int POLICY>
__global__ void __launch_bounds__(PNT) read_probe_kernel(const unsigned char *src, int64_t bytes, int64_t span,
                                                         unsigned *sink) {
    const int64_t b0 = (int64_t)blockIdx.x * span;
    const int64_t b1 = b0 + span < bytes ? b0 + span : bytes;
    unsigned acc = 0;
    constexpr int64_t STEP = (int64_t)PNT * 16 * UNROLL;
    for (int64_t o = b0; o < b1; o += STEP) {
        // the span and the buffer are whole multiples of 16 bytes; a span's
        // last round may stop early (out-of-range lanes read as zero)
        const rsrc_t r = make_rsrc(src + o, b1 - o);
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 r, (unsigned)((u * PNT + (int)threadIdx.x) * 16), 0, POLICY));
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // one word per work-group: lane 0 of each wave folds its wave's words
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_xor(sink + blockIdx.x, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

hipError_t launch_read_probe(const void *src, int64_t bytes, int wgs, int unroll, bool nontemporal, unsigned *sink,
                             hipStream_t s) {
    if (bytes <= 0 || bytes % 16 != 0 || wgs <= 0) return hipErrorInvalidValue;
    const int64_t span = cdiv(cdiv(bytes, wgs), 16) * 16;
    if (span >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const auto *p = (const unsigned char *)src;
#define LL_PROBE(U)                                                                                                   \
    if (unroll == U) {                                                                                                \
        if (nontemporal)                                                                                              \
            hipLaunchKernelGGL((read_probe_kernel<U, 2>), dim3(wgs), dim3(PNT), 0, s, p, bytes, span, sink);          \
        else                                                                                                          \
            hipLaunchKernelGGL((read_probe_kernel<U, 0>), dim3(wgs), dim3(PNT), 0, s, p, bytes, span, sink);          \
        return hipGetLastError();                                                                                     \
    }
    LL_PROBE(4)
    LL_PROBE(8)
    LL_PROBE(16)
#undef LL_PROBE
    return hipErrorInvalidValue;
}

}  // namespace ll
