// Host-side runtime pieces shared by the launchers: the compute-unit count of
// a device, the opt-in stream-ordered workspace pool, debug reporting and the
// segment-length knob.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;                       // guards the two per-device caches
hipMemPool_t g_pools[kMaxDevices] = {};
int g_cu_count[kMaxDevices] = {};
std::atomic<int64_t> g_forced_segment{0};

// A pool per device whose freed blocks go back to the device at the next
// synchronisation (release threshold 0): nothing stays reserved between calls.
hipMemPool_t workspace_pool(int dev)
{
    std::lock_guard<std::mutex> lk(g_mutex);
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    if (!g_pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        hipError_t e = hipMemPoolCreate(&p, &props);
        report("hipMemPoolCreate", e);
        if (e != hipSuccess) {
            (void)hipGetLastError();  // this call's own failure, not the caller's
            return nullptr;
        }
        uint64_t keep = 0;
        e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
        report("hipMemPoolSetAttribute", e);
        if (e != hipSuccess) (void)hipGetLastError();
        g_pools[dev] = p;
    }
    return g_pools[dev];
}

}  // namespace

bool debug_enabled()
{
    static const bool on = std::getenv("KDA_DEBUG") != nullptr;
    return on;
}

void report(const char* what, hipError_t e)
{
    if (debug_enabled() && e != hipSuccess)
        std::fprintf(stderr, "kda: %s: %s\n", what, hipGetErrorString(e));
}

int cu_count(int dev)
{
    std::lock_guard<std::mutex> lk(g_mutex);
    if (dev < 0 || dev >= kMaxDevices) return 256;
    if (!g_cu_count[dev]) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0) {
            (void)hipGetLastError();
            c = 256;
        }
        g_cu_count[dev] = c;
    }
    return g_cu_count[dev];
}

hipError_t StreamWorkspace::acquire(size_t bytes, hipStream_t s)
{
    (void)release();
    if (bytes == 0) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    hipMemPool_t pool = workspace_pool(dev);
    if (!pool) return hipErrorOutOfMemory;
    void* p = nullptr;
    e = hipMallocFromPoolAsync(&p, bytes, pool, s);
    report("hipMallocFromPoolAsync", e);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // reported to the caller as a status instead
        return e;
    }
    ptr = p;
    stream = s;
    return hipSuccess;
}

hipError_t StreamWorkspace::release()
{
    if (!ptr) return hipSuccess;
    const hipError_t e = hipFreeAsync(ptr, stream);
    report("hipFreeAsync", e);
    ptr = nullptr;
    return e;
}

int64_t forced_segment() { return g_forced_segment.load(std::memory_order_relaxed); }

void set_forced_segment(int64_t tokens) { g_forced_segment.store(tokens, std::memory_order_relaxed); }

}  // namespace kda
