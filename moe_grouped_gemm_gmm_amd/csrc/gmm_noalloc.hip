// Library-owned scratch for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// workspace of gmm_fp8_fwd_noalloc lives in a file-scope device array
// instead of a caller buffer.
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in symbol): on the first call on a device, with
// that device current, hipGetSymbolAddress gives the device address, which
// is kept per device and is what kernels receive.  Every call on a device
// shares that device's array and finds the last call's contents there;
// calls that overlap on one device race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gmm_launch.hpp"

namespace gmm {

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices] = {};
hipError_t g_err[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_err[dev] = r;
        g_ptr[dev] = r == hipSuccess ? p : nullptr;
    });
    if (g_err[dev] != hipSuccess) return g_err[dev];
    *ptr = g_ptr[dev];
    *bytes = kNoallocScratchBytes;
    return hipSuccess;
}

}  // namespace gmm
