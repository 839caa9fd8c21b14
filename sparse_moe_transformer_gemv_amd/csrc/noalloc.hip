// noalloc.hip -- the static device scratch behind flint_moe_forward_noalloc,
// for callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is one file-scope device array per GPU, loaded with the code
// object and held until the process ends.  In host code its name is a
// host-side stand-in, not a device address: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept here, and only that address is ever handed to kernels or copies.
#include <mutex>

#include "flint_internal.hpp"

namespace flint {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device (null: not set up)
}  // namespace

hipError_t scratch_for_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace flint
