// Host-only argument checks of the C ABI (declared in include/litelinear.h
// and check.hpp).  No HIP calls: the forward entry points run them before
// touching the device, and the host sanitizer build compiles this file on
// its own.
#include "check.hpp"

namespace ll {

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

litelinear_status_t check_args_ld(const void *x, int64_t ldx, const void *A, const void *B, const void *Q,
                                  const void *bias, const void *y, int64_t M, int64_t in, int64_t out, int64_t r,
                                  int y_bytes_per_elem, bool glu) {
    const int64_t lim = (int64_t)1 << 40;
    if (M < 0 || in < 0 || out < 0 || r < 0) return LITELINEAR_ERR_INVALID_ARG;
    if (ldx < in || ldx > lim || (double)M * (double)ldx > 4.0e18) return LITELINEAR_ERR_INVALID_ARG;
    if (y_bytes_per_elem != 2 && y_bytes_per_elem != 4) return LITELINEAR_ERR_INVALID_ARG;
    if (M > lim || in > lim || out > lim || r > lim) return LITELINEAR_ERR_INVALID_ARG;
    if ((double)M * (double)in > 4.0e18 || (double)M * (double)out > 1.0e18 ||
        (double)out * (double)in > 4.0e18 || (double)r * (double)(in + out) > 4.0e18)
        return LITELINEAR_ERR_INVALID_ARG;
    if (M == 0 || out == 0) return LITELINEAR_OK;  // nothing to compute
    if (!y) return LITELINEAR_ERR_INVALID_ARG;
    if (in > 0 && (!x || !Q)) return LITELINEAR_ERR_INVALID_ARG;
    if (r > 0 && (!A || (in > 0 && !B))) return LITELINEAR_ERR_INVALID_ARG;
    if (in % 16 != 0) return LITELINEAR_ERR_UNSUPPORTED;
    if (in > 0 && (!aligned(x, 16) || !aligned(Q, 16) || ldx % 8 != 0)) return LITELINEAR_ERR_UNSUPPORTED;
    if (r > 0 && in > 0 && !aligned(B, 16)) return LITELINEAR_ERR_UNSUPPORTED;
    if (r > 0 && !aligned(A, 2)) return LITELINEAR_ERR_UNSUPPORTED;
    if (bias && !aligned(bias, 2)) return LITELINEAR_ERR_UNSUPPORTED;
    if (!aligned(y, (uintptr_t)y_bytes_per_elem)) return LITELINEAR_ERR_UNSUPPORTED;
    // the gated epilogue writes half as many columns as Q has rows
    if (glu && out % 2 != 0) return LITELINEAR_ERR_INVALID_ARG;
    const uint64_t ny = (uint64_t)M * (uint64_t)(glu ? out / 2 : out) * (uint64_t)y_bytes_per_elem;
    // x's extent: M - 1 row strides and one row
    const uint64_t nx = in > 0 ? ((uint64_t)(M - 1) * (uint64_t)ldx + (uint64_t)in) * 2 : 0;
    if (overlaps(y, ny, x, nx) || overlaps(y, ny, Q, (uint64_t)out * in) ||
        (r > 0 && (overlaps(y, ny, A, (uint64_t)out * r * 2) || overlaps(y, ny, B, (uint64_t)r * in * 2))) ||
        overlaps(y, ny, bias, (uint64_t)out * 2))
        return LITELINEAR_ERR_INVALID_ARG;
    return LITELINEAR_OK;
}

}  // namespace ll

extern "C" litelinear_status_t litelinear_check_args(const void *x, const void *A, const void *B, const void *Q,
                                                     const void *bias, const void *y, int64_t M, int64_t in,
                                                     int64_t out, int64_t r, int y_bytes_per_elem) {
    return ll::check_args_ld(x, in, A, B, Q, bias, y, M, in, out, r, y_bytes_per_elem);
}
