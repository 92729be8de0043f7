// Device-side precondition checks, run before a call's kernels when KDA_DEBUG
// is set in the environment (the debug mode of the C ABI; it synchronises).
//
// The preconditions are those the header documents but cannot check on the
// host without a synchronisation, because the data are in device memory:
//  - every log forgetting factor is finite and <= 0 (the gate alpha =
//    exp(log alpha) is a forgetting factor in (0, 1]; "Kimi K3 -- the
//    architecture and infrastructure, explained", section "Kimi Delta
//    Attention: the load-bearing choice", gives one such factor per channel);
//    for the raw-projection calls, every gate logit is finite;
//  - cu_seqlens starts at 0, never decreases and ends at T_total.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kda_internal.hpp"

namespace kda {
namespace {

// One violation word per device, found through hipGetSymbolAddress (the
// host-side name of a __device__ variable is not a device address).
__device__ unsigned int g_violations;

__global__ void clear_kernel(unsigned int* flags) { *flags = 0u; }

__global__ __launch_bounds__(256) void gate_kernel(const float* log_alpha, int64_t n, int raw,
                                                   unsigned int* flags)
{
    bool bad = false;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = log_alpha[i];
        // NaN fails both comparisons; +-inf fails the magnitude test
        const bool finite = x == x && x <= 3.4028235e38f && x >= -3.4028235e38f;
        bad |= !finite || (!raw && x > 0.f);
    }
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flags, kViolationGate);
}

__global__ __launch_bounds__(256) void seqlens_kernel(const int32_t* cu, int64_t n_seq,
                                                      int64_t T_total, unsigned int* flags)
{
    unsigned int bad = 0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_seq; i += stride)
        if (cu[i + 1] < cu[i]) bad |= kViolationOrder;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (cu[0] != 0) bad |= kViolationStart;
        if (static_cast<int64_t>(cu[n_seq]) != T_total) bad |= kViolationEnd;
    }
    if (bad) atomicOr(flags, bad);
}

std::mutex g_check_mutex;  // one check at a time shares the violation word

}  // namespace

hipError_t check_preconditions(const float* log_alpha, int64_t n_gates, bool raw,
                               const int32_t* cu_seqlens, int64_t n_seq, int64_t T_total,
                               hipStream_t stream, unsigned int* violations)
{
    *violations = 0;
    std::lock_guard<std::mutex> lk(g_check_mutex);
    unsigned int* flags = nullptr;
    hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&flags), HIP_SYMBOL(g_violations));
    report("hipGetSymbolAddress", e);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(1), 0, stream, flags);
    if (log_alpha && n_gates > 0) {
        const int64_t blocks = (n_gates + 255) / 256;
        hipLaunchKernelGGL(gate_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                           dim3(256), 0, stream, log_alpha, n_gates, raw ? 1 : 0, flags);
    }
    if (cu_seqlens) {
        const int64_t blocks = (n_seq + 255) / 256;
        hipLaunchKernelGGL(seqlens_kernel,
                           dim3(static_cast<unsigned>(blocks < 1 ? 1 : blocks < 4096 ? blocks : 4096)),
                           dim3(256), 0, stream, cu_seqlens, n_seq, T_total, flags);
    }
    e = hipGetLastError();
    report("precondition check launch", e);
    if (e != hipSuccess) return e;
    unsigned int host = 0;
    e = hipMemcpyAsync(&host, flags, sizeof(host), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    report("precondition check copy", e);
    if (e != hipSuccess) return e;
    *violations = host;
    return hipSuccess;
}

}  // namespace kda
