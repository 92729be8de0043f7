// The fixed scratch of kda_prefill_noalloc: a file-scope device array that
// every call on a device shares, for callers that cannot allocate device
// memory (code under graph capture, serving loops that forbid allocation).
//
// The host-side name of a __device__ array is not a device address: the
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and only that pointer is handed to the kernels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kda_internal.hpp"

namespace kda {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr)
{
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    report("hipGetDevice", e);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        report("hipGetSymbolAddress(scratch)", e);
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
