// Fixed device scratch for litelinear_forward_noalloc: the workspace of the
// forward (T' blocks, K-slice partial sums, counters, a padded copy of A,
// e4m3fn activations) carved out of one file-scope device array instead of
// memory the library allocates, for callers that cannot allocate (code under
// graph capture, tight serving loops).
//
// Each device that the library loads on holds its own copy of the array
// until the process ends.  Host code never uses the array's name as an
// address (on the host it only stands in for the symbol): scratch_init()
// looks the device address up once per device, with that device current,
// and every later use goes through that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

static __device__ __align__(256) unsigned char scratch[ll::kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

}  // namespace

namespace ll {

hipError_t scratch_init(int device, void **ptr) {
    *ptr = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device) return hipErrorInvalidDevice;  // the caller makes the device current
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return e != hipSuccess ? e : hipErrorInvalidSymbol;
        g_scratch[device] = p;
    }
    *ptr = g_scratch[device];
    return hipSuccess;
}

}  // namespace ll
