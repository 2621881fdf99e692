// Host-only argument checks of the C ABI (check.cpp): plain C++ with no HIP
// calls, so that they also build on their own for a host sanitizer run.
#pragma once

#include <stdint.h>

#include "litelinear.h"

namespace ll {

// [a, a + na) and [b, b + nb) overlap (a null pointer or an empty range never does).
bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb);
bool aligned(const void *p, uintptr_t n);

// litelinear_check_args() for x rows ldx elements apart; glu: the gated
// epilogue (y has out / 2 columns, out must be even).
litelinear_status_t check_args_ld(const void *x, int64_t ldx, const void *A, const void *B, const void *Q,
                                  const void *bias, const void *y, int64_t M, int64_t in, int64_t out, int64_t r,
                                  int y_bytes_per_elem, bool glu = false);

}  // namespace ll
