// The library's own device scratch: split-K partial results of the
// allocation-free decode entry point, for callers that cannot allocate
// device memory (code under graph capture, serving loops that forbid it).
//
// One file-scope array per device, held from library load until the
// process ends.  Host code never uses the array's name as an address (on
// the host it names a stand-in): the first call on a device, with that
// device current, looks up the device's own copy with hipGetSymbolAddress,
// and every later call on that device reuses the address.

#include <hip/hip_runtime.h>

#include <mutex>

#include "pbq_internal.h"

namespace pbq {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace pbq
