// C ABI of libkda.so (declared in include/kda.h): host-side validation, the
// choice of plan and workspace, then asynchronous launches on the caller's
// stream.  Every check happens before a launch, so that on error nothing is
// enqueued; nothing here synchronises, except the KDA_DEBUG precondition
// checks.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

#include "kda_internal.hpp"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 46;  // keeps every index product in int64

bool misaligned(const void* p, uintptr_t a = 16) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

kda_status check_dtype(kda_dtype d)
{
    return (d == KDA_F32 || d == KDA_BF16) ? KDA_OK : KDA_ERR_DTYPE;
}

kda_status check_dims(int64_t H, int64_t d_k, int64_t d_v)
{
    if (H < 1 || d_k < 1 || d_v < 1) return KDA_ERR_SHAPE;
    // offsets within a 64-token chunk are 32-bit in the kernels
    if (H > kda::kMaxHeads) return KDA_ERR_SHAPE;
    if (d_k != kda::kDim || d_v != kda::kDim) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

// rows * H * 128 must stay far from int64 overflow and grid limits.
kda_status check_rows(int64_t rows, int64_t H)
{
    if (rows < 0) return KDA_ERR_SHAPE;
    if (rows > 0 && (rows > kMaxElems / H / kda::kDim)) return KDA_ERR_SHAPE;
    return KDA_OK;
}

kda_status check_ptrs(std::initializer_list<const void*> required,
                      std::initializer_list<const void*> optional)
{
    for (const void* p : required)
        if (!p) return KDA_ERR_NULL;
    for (const void* p : required)
        if (misaligned(p)) return KDA_ERR_ALIGN;
    for (const void* p : optional)
        if (p && misaligned(p)) return KDA_ERR_ALIGN;
    return KDA_OK;
}

// Byte ranges [p, p + n) of device buffers; NULL or empty ranges overlap nothing.
struct Span {
    const void* p;
    uint64_t n;
};
bool overlap(Span a, Span b)
{
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
    return x < y + b.n && y < x + a.n;
}

// A caller-owned workspace is `bytes` bytes at a 256-byte aligned `ws` (NULL
// when bytes is 0); KDA_WORKSPACE_AUTO asks the library for one (ws NULL).
kda_status check_workspace(const void* ws, int64_t bytes)
{
    if (bytes == KDA_WORKSPACE_AUTO) return ws ? KDA_ERR_WORKSPACE : KDA_OK;
    if (bytes < 0) return KDA_ERR_WORKSPACE;
    if (bytes > 0 && !ws) return KDA_ERR_NULL;
    if (ws && misaligned(ws, 256)) return KDA_ERR_ALIGN;
    return KDA_OK;
}

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// An unread HIP error of the calling thread (left by an earlier call of the
// caller's) stays for the caller to read: the call enqueues nothing.  After
// this check, hipGetLastError() after a launch reports that launch only.
kda_status no_pending_error()
{
    const hipError_t e = hipPeekAtLastError();
    kda::report("an earlier HIP error is pending; nothing enqueued", e);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// The current device and its compute units (the plans are sized by them).
kda_status current_cus(int* n_cu)
{
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    kda::report("hipGetDevice", e);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // this call's own failure, reported as a status
        return KDA_ERR_HIP;
    }
    *n_cu = kda::cu_count(dev);
    return KDA_OK;
}

// KDA_DEBUG: the device-side preconditions, checked before anything else is
// enqueued (this synchronises the stream).
kda_status debug_check(const float* log_alpha, int64_t n_gates, bool raw, const int32_t* cu,
                       int64_t n_seq, int64_t T_total, hipStream_t stream)
{
    if (!kda::debug_enabled()) return KDA_OK;
    unsigned int bad = 0;
    const hipError_t e =
        kda::check_preconditions(log_alpha, n_gates, raw, cu, n_seq, T_total, stream, &bad);
    if (e != hipSuccess) return KDA_ERR_HIP;
    return bad ? KDA_ERR_PRECONDITION : KDA_OK;
}

// bf16 inputs take the chunked matrix-core kernel, except sequences of at most
// kShortPrefill tokens; fp32 inputs (whose q and k are not exact in bf16) and
// those short sequences take the register-resident token-by-token kernel.
bool prefill_uses_scan(kda_dtype in_dtype, bool packed, int64_t T, int64_t T_total)
{
    const int64_t longest = packed ? T_total : T;
    return in_dtype == KDA_BF16 && longest > kda::kShortPrefill;
}

// The fastest plan whose workspace fits `bytes` (the fastest of all for
// KDA_WORKSPACE_AUTO); the tier-2 plan needs none, so one always fits.
kda::PrefillPlan fitting_plan(bool packed, int64_t n_seq, int64_t T, int64_t T_total, int64_t H,
                              int n_cu, int64_t bytes)
{
    const int64_t forced = kda::forced_segment();
    for (int tier = 0; tier < 2; ++tier) {
        const kda::PrefillPlan p = kda::plan_prefill_scan(packed, n_seq, T, T_total, H, n_cu, forced, tier);
        if (bytes == KDA_WORKSPACE_AUTO || static_cast<int64_t>(p.ws_bytes) <= bytes) return p;
    }
    return kda::plan_prefill_scan(packed, n_seq, T, T_total, H, n_cu, forced, 2);
}

kda_status run_prefill(const void* q, const void* k, const void* v, const void* beta,
                       const float* log_alpha, const int32_t* cu_seqlens, int64_t n_seq, int64_t T,
                       int64_t T_total, int64_t H, const kda::StateRefs& st, float* o,
                       kda_dtype in_dtype, bool raw, void* workspace, int64_t workspace_bytes,
                       hipStream_t stream)
{
    const bool packed = cu_seqlens != nullptr;
    const int64_t rows = packed ? T_total : n_seq * T;
    kda_status s;
    if ((s = no_pending_error()) != KDA_OK) return s;
    if ((s = debug_check(rows > 0 ? log_alpha : nullptr, rows * H * kda::kDim, raw, cu_seqlens,
                         n_seq, T_total, stream)) != KDA_OK)
        return s;
    if (!prefill_uses_scan(in_dtype, packed, T, T_total))
        return from_hip(kda::launch_prefill_recurrent(q, k, v, beta, log_alpha, cu_seqlens, n_seq, T,
                                                      H, st, o, in_dtype == KDA_BF16, raw, 0, stream));
    int n_cu = 0;
    if ((s = current_cus(&n_cu)) != KDA_OK) return s;
    const kda::PrefillPlan plan = fitting_plan(packed, n_seq, T, T_total, H, n_cu, workspace_bytes);
    kda::StreamWorkspace lease;
    void* ws = workspace;
    if (workspace_bytes == KDA_WORKSPACE_AUTO && plan.ws_bytes > 0) {
        if (lease.acquire(plan.ws_bytes, stream) != hipSuccess) return KDA_ERR_WORKSPACE;
        ws = lease.ptr;
    }
    // bf16 packed: short sequences token by token, the others chunked.  Each
    // kernel skips the other's sequences (packed lengths are on the device).
    hipError_t e = kda::launch_prefill_scan(q, k, v, beta, log_alpha, cu_seqlens, n_seq, T, H, st, o,
                                            raw, packed ? kda::kShortPrefill : 0, plan, ws, n_cu,
                                            stream);
    if (e == hipSuccess && packed)
        e = kda::launch_prefill_recurrent(q, k, v, beta, log_alpha, cu_seqlens, n_seq, T, H, st, o,
                                          true, raw, kda::kShortPrefill, stream);
    const hipError_t f = lease.release();
    return from_hip(e != hipSuccess ? e : f);
}

kda::StateRefs plain_states(const float* initial_state, float* final_state)
{
    kda::StateRefs st;
    st.init = initial_state;
    st.fin = final_state;
    return st;
}

// pool entries of H * 128 * 128 floats must stay far from int64 overflow
bool pool_too_big(int64_t n_pool, int64_t H)
{
    return n_pool > kMaxElems / H / (int64_t(kda::kDim) * kda::kDim);
}

kda_status check_dense(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v, kda_dtype in_dtype)
{
    kda_status st;
    if ((st = check_dtype(in_dtype)) != KDA_OK) return st;
    if ((st = check_dims(H, d_k, d_v)) != KDA_OK) return st;
    if (B < 0 || T < 0) return KDA_ERR_SHAPE;
    if (B > 0 && T > kMaxElems / B) return KDA_ERR_SHAPE;
    if ((st = check_rows(B * T, H)) != KDA_OK) return st;
    if (B > int64_t(1) << 24 || B * H > int64_t(1) << 30) return KDA_ERR_SHAPE;
    return KDA_OK;
}

kda_status check_packed(int64_t N, int64_t T_total, int64_t H, int64_t d_k, int64_t d_v,
                        kda_dtype in_dtype)
{
    kda_status st;
    if ((st = check_dtype(in_dtype)) != KDA_OK) return st;
    if ((st = check_dims(H, d_k, d_v)) != KDA_OK) return st;
    if (N < 0 || T_total < 0) return KDA_ERR_SHAPE;
    // cu_seqlens holds int32 row indices
    if (T_total > INT32_MAX || N > int64_t(1) << 24 || N * H > int64_t(1) << 30) return KDA_ERR_SHAPE;
    return check_rows(T_total, H);
}

kda_status prefill_impl(const void* q, const void* k, const void* v, const void* beta,
                        const float* log_alpha, const float* initial_state, float* o,
                        float* final_state, int64_t B, int64_t T, int64_t H, int64_t d_k,
                        int64_t d_v, kda_dtype in_dtype, bool raw, void* workspace,
                        int64_t workspace_bytes, void* stream)
{
    kda_status st;
    if ((st = check_dense(B, T, H, d_k, d_v, in_dtype)) != KDA_OK) return st;
    if ((st = check_workspace(workspace, workspace_bytes)) != KDA_OK) return st;
    if (B == 0) return KDA_OK;
    if (T > 0) {
        if ((st = check_ptrs({q, k, v, beta, log_alpha, o}, {initial_state, final_state})) != KDA_OK)
            return st;
    } else if ((st = check_ptrs({}, {initial_state, final_state})) != KDA_OK) {
        return st;
    }
    if (T == 0 && !final_state) return KDA_OK;
    return run_prefill(q, k, v, beta, log_alpha, nullptr, B, T, B * T, H,
                       plain_states(initial_state, final_state), o, in_dtype, raw, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream));
}

kda_status varlen_impl(const void* q, const void* k, const void* v, const void* beta,
                       const float* log_alpha, const int32_t* cu_seqlens, int64_t N,
                       int64_t T_total, const float* initial_state, float* o, float* final_state,
                       int64_t H, int64_t d_k, int64_t d_v, kda_dtype in_dtype, bool raw,
                       void* workspace, int64_t workspace_bytes, void* stream)
{
    kda_status st;
    if ((st = check_packed(N, T_total, H, d_k, d_v, in_dtype)) != KDA_OK) return st;
    if ((st = check_workspace(workspace, workspace_bytes)) != KDA_OK) return st;
    if (N == 0) return KDA_OK;
    if (!cu_seqlens) return KDA_ERR_NULL;
    if (misaligned(cu_seqlens)) return KDA_ERR_ALIGN;
    if (T_total > 0) {
        if ((st = check_ptrs({q, k, v, beta, log_alpha, o}, {initial_state, final_state})) != KDA_OK)
            return st;
    } else if ((st = check_ptrs({}, {initial_state, final_state})) != KDA_OK) {
        return st;
    }
    if (T_total == 0 && !final_state) return KDA_OK;
    return run_prefill(q, k, v, beta, log_alpha, cu_seqlens, N, 0, T_total, H,
                       plain_states(initial_state, final_state), o, in_dtype, raw, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream));
}

kda_status decode_impl(const void* q, const void* k, const void* v, const void* beta,
                       const float* log_alpha, float* state, float* o, int64_t N, int64_t H,
                       int64_t d_k, int64_t d_v, kda_dtype in_dtype, bool raw, void* stream)
{
    kda_status st;
    if ((st = check_dtype(in_dtype)) != KDA_OK) return st;
    if ((st = check_dims(H, d_k, d_v)) != KDA_OK) return st;
    if (N < 0) return KDA_ERR_SHAPE;
    if (N > int64_t(1) << 24 || N * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (N == 0) return KDA_OK;
    if ((st = check_ptrs({q, k, v, beta, log_alpha, state, o}, {})) != KDA_OK) return st;
    if ((st = no_pending_error()) != KDA_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = debug_check(log_alpha, N * H * kda::kDim, raw, nullptr, 0, 0, s)) != KDA_OK) return st;
    return from_hip(kda::launch_decode_step(q, k, v, beta, log_alpha, state, nullptr, 0, o, N * H,
                                            H, in_dtype == KDA_BF16, raw, s));
}

kda_status backward_sizes(bool packed, int64_t n_seq, int64_t T, int64_t T_total, int64_t H,
                          int64_t d_k, int64_t d_v, kda_dtype in_dtype)
{
    return packed ? check_packed(n_seq, T_total, H, d_k, d_v, in_dtype)
                  : check_dense(n_seq, T, H, d_k, d_v, in_dtype);
}

kda_status backward_impl(const void* q, const void* k, const void* v, const void* beta,
                         const float* log_alpha, const int32_t* cu_seqlens, int64_t n_seq,
                         int64_t T, int64_t T_total, const float* initial_state, const float* d_o,
                         const float* d_final_state, float* dq, float* dk, float* dv, float* dbeta,
                         float* dlog_alpha, float* d_initial_state, int64_t H, int64_t d_k,
                         int64_t d_v, kda_dtype in_dtype, void* workspace, int64_t workspace_bytes,
                         void* stream)
{
    const bool packed = cu_seqlens != nullptr;
    kda_status st;
    if ((st = backward_sizes(packed, n_seq, T, T_total, H, d_k, d_v, in_dtype)) != KDA_OK) return st;
    if ((st = check_workspace(workspace, workspace_bytes)) != KDA_OK) return st;
    if (n_seq == 0) return KDA_OK;
    if (packed && misaligned(cu_seqlens)) return KDA_ERR_ALIGN;
    const int64_t rows = packed ? T_total : n_seq * T;
    if (rows > 0) {
        if ((st = check_ptrs({q, k, v, beta, log_alpha, d_o, dq, dk, dv, dbeta, dlog_alpha},
                             {initial_state, d_final_state, d_initial_state})) != KDA_OK)
            return st;
        // the gradient buffers are written while the inputs are still read (and
        // hold intermediates): no output may overlap an input or another output,
        // except d_initial_state == d_final_state
        const uint64_t ie = in_dtype == KDA_BF16 ? 2 : 4;
        const uint64_t vec = static_cast<uint64_t>(rows) * H * kda::kDim, sc = static_cast<uint64_t>(rows) * H;
        const uint64_t stb = static_cast<uint64_t>(n_seq) * H * kda::kStateFloats * 4;
        const Span outs[] = {{dq, vec * 4}, {dk, vec * 4}, {dv, vec * 4}, {dlog_alpha, vec * 4},
                             {dbeta, sc * 4}, {d_initial_state, stb}};
        const Span ins[] = {{q, vec * ie}, {k, vec * ie}, {v, vec * ie}, {beta, sc * ie},
                            {log_alpha, vec * 4}, {d_o, vec * 4}, {initial_state, stb},
                            {d_final_state, stb}};
        for (size_t i = 0; i < 6; ++i) {
            for (size_t j = 0; j < i; ++j)
                if (overlap(outs[i], outs[j])) return KDA_ERR_OVERLAP;
            for (const Span& in : ins) {
                if (i == 5 && in.p == d_final_state && d_initial_state == d_final_state) continue;
                if (overlap(outs[i], in)) return KDA_ERR_OVERLAP;
            }
        }
    } else if ((st = check_ptrs({}, {initial_state, d_final_state, d_initial_state})) != KDA_OK) {
        return st;
    }
    if (rows == 0 && !d_initial_state) return KDA_OK;
    if ((st = no_pending_error()) != KDA_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = debug_check(rows > 0 ? log_alpha : nullptr, rows * H * kda::kDim, false, cu_seqlens,
                          n_seq, T_total, s)) != KDA_OK)
        return st;
    const kda::BackwardPlan plan =
        kda::plan_backward(packed, n_seq, T, T_total, H, in_dtype == KDA_BF16);
    kda::StreamWorkspace lease;
    void* ws = workspace;
    if (workspace_bytes == KDA_WORKSPACE_AUTO) {
        if (plan.ws_bytes > 0 && lease.acquire(plan.ws_bytes, s) != hipSuccess) return KDA_ERR_WORKSPACE;
        ws = lease.ptr;
    } else if (static_cast<int64_t>(plan.ws_bytes) > workspace_bytes) {
        return KDA_ERR_WORKSPACE;
    }
    const hipError_t e = kda::launch_backward(q, k, v, beta, log_alpha, d_o, cu_seqlens, n_seq, T, H,
                                              initial_state, d_final_state, dq, dk, dv, dbeta,
                                              dlog_alpha, d_initial_state, in_dtype == KDA_BF16, plan,
                                              ws, s);
    const hipError_t f = lease.release();
    return from_hip(e != hipSuccess ? e : f);
}

kda_status prefill_size(bool packed, int64_t n_seq, int64_t T, int64_t T_total, int64_t H,
                        int64_t d_k, int64_t d_v, kda_dtype in_dtype, kda_plan plan, int64_t* bytes)
{
    if (!bytes) return KDA_ERR_NULL;
    *bytes = 0;
    kda_status st = packed ? check_packed(n_seq, T_total, H, d_k, d_v, in_dtype)
                           : check_dense(n_seq, T, H, d_k, d_v, in_dtype);
    if (st != KDA_OK) return st;
    if (plan != KDA_PLAN_FULL && plan != KDA_PLAN_SEGMENTS && plan != KDA_PLAN_UNSEGMENTED)
        return KDA_ERR_SHAPE;
    if (n_seq == 0 || !prefill_uses_scan(in_dtype, packed, T, T_total)) return KDA_OK;
    int n_cu = 0;
    if ((st = current_cus(&n_cu)) != KDA_OK) return st;
    *bytes = static_cast<int64_t>(kda::plan_prefill_scan(packed, n_seq, T, packed ? T_total : n_seq * T,
                                                         H, n_cu, kda::forced_segment(),
                                                         static_cast<int>(plan)).ws_bytes);
    return KDA_OK;
}

kda_status backward_size(bool packed, int64_t n_seq, int64_t T, int64_t T_total, int64_t H,
                         int64_t d_k, int64_t d_v, kda_dtype in_dtype, int64_t* bytes)
{
    if (!bytes) return KDA_ERR_NULL;
    *bytes = 0;
    kda_status st = backward_sizes(packed, n_seq, T, T_total, H, d_k, d_v, in_dtype);
    if (st != KDA_OK) return st;
    if (n_seq == 0) return KDA_OK;
    *bytes = static_cast<int64_t>(
        kda::plan_backward(packed, n_seq, T, T_total, H, in_dtype == KDA_BF16).ws_bytes);
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prefill(const void* q, const void* k, const void* v, const void* beta,
                       const float* log_alpha, const float* initial_state, float* o,
                       float* final_state, int64_t B, int64_t T, int64_t H, int64_t d_k,
                       int64_t d_v, kda_dtype in_dtype, void* workspace, int64_t workspace_bytes,
                       void* stream)
{
    return prefill_impl(q, k, v, beta, log_alpha, initial_state, o, final_state, B, T, H, d_k, d_v,
                        in_dtype, false, workspace, workspace_bytes, stream);
}

kda_status kda_prefill_raw(const void* q, const void* k, const void* v, const void* beta,
                           const float* log_alpha, const float* initial_state, float* o,
                           float* final_state, int64_t B, int64_t T, int64_t H, int64_t d_k,
                           int64_t d_v, kda_dtype in_dtype, void* workspace,
                           int64_t workspace_bytes, void* stream)
{
    return prefill_impl(q, k, v, beta, log_alpha, initial_state, o, final_state, B, T, H, d_k, d_v,
                        in_dtype, true, workspace, workspace_bytes, stream);
}

kda_status kda_prefill_noalloc(const void* q, const void* k, const void* v, const void* beta,
                               const float* log_alpha, const float* initial_state, float* o,
                               float* final_state, int64_t B, int64_t T, int64_t H, int64_t d_k,
                               int64_t d_v, kda_dtype in_dtype, void* stream)
{
    kda_status st;
    if ((st = check_dense(B, T, H, d_k, d_v, in_dtype)) != KDA_OK) return st;
    if (B == 0 || T == 0) {
        // nothing segmented: the plain call, which needs no workspace here
        return prefill_impl(q, k, v, beta, log_alpha, initial_state, o, final_state, B, T, H, d_k,
                            d_v, in_dtype, false, nullptr, 0, stream);
    }
    // the pointers are validated before anything touches the device
    if ((st = check_ptrs({q, k, v, beta, log_alpha, o}, {initial_state, final_state})) != KDA_OK)
        return st;
    const int64_t limit = static_cast<int64_t>(kda::kNoallocScratchBytes);
    if (prefill_uses_scan(in_dtype, false, T, B * T)) {
        // refuse what the scratch cannot hold without falling back to the
        // unsegmented plan: the segments plan must fit
        int n_cu = 0;
        if ((st = current_cus(&n_cu)) != KDA_OK) return st;
        const kda::PrefillPlan seg =
            kda::plan_prefill_scan(false, B, T, B * T, H, n_cu, kda::forced_segment(), 1);
        if (static_cast<int64_t>(seg.ws_bytes) > limit) return KDA_ERR_WORKSPACE;
    }
    void* scratch = nullptr;
    if (kda::noalloc_scratch(&scratch) != hipSuccess) {
        (void)hipGetLastError();  // the lookup's own failure, reported as a status
        return KDA_ERR_HIP;
    }
    return prefill_impl(q, k, v, beta, log_alpha, initial_state, o, final_state, B, T, H, d_k, d_v,
                        in_dtype, false, scratch, limit, stream);
}

kda_status kda_varlen_prefill(const void* q, const void* k, const void* v, const void* beta,
                              const float* log_alpha, const int32_t* cu_seqlens, int64_t N,
                              int64_t T_total, const float* initial_state, float* o,
                              float* final_state, int64_t H, int64_t d_k, int64_t d_v,
                              kda_dtype in_dtype, void* workspace, int64_t workspace_bytes,
                              void* stream)
{
    return varlen_impl(q, k, v, beta, log_alpha, cu_seqlens, N, T_total, initial_state, o,
                       final_state, H, d_k, d_v, in_dtype, false, workspace, workspace_bytes, stream);
}

kda_status kda_varlen_prefill_raw(const void* q, const void* k, const void* v, const void* beta,
                                  const float* log_alpha, const int32_t* cu_seqlens, int64_t N,
                                  int64_t T_total, const float* initial_state, float* o,
                                  float* final_state, int64_t H, int64_t d_k, int64_t d_v,
                                  kda_dtype in_dtype, void* workspace, int64_t workspace_bytes,
                                  void* stream)
{
    return varlen_impl(q, k, v, beta, log_alpha, cu_seqlens, N, T_total, initial_state, o,
                       final_state, H, d_k, d_v, in_dtype, true, workspace, workspace_bytes, stream);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* beta,
                           const float* log_alpha, float* state, float* o, int64_t N, int64_t H,
                           int64_t d_k, int64_t d_v, kda_dtype in_dtype, void* stream)
{
    return decode_impl(q, k, v, beta, log_alpha, state, o, N, H, d_k, d_v, in_dtype, false, stream);
}

kda_status kda_decode_step_raw(const void* q, const void* k, const void* v, const void* beta,
                               const float* log_alpha, float* state, float* o, int64_t N, int64_t H,
                               int64_t d_k, int64_t d_v, kda_dtype in_dtype, void* stream)
{
    return decode_impl(q, k, v, beta, log_alpha, state, o, N, H, d_k, d_v, in_dtype, true, stream);
}

kda_status kda_varlen_prefill_slots(const void* q, const void* k, const void* v, const void* beta,
                                    const float* log_alpha, const int32_t* cu_seqlens, int64_t N,
                                    int64_t T_total, float* state_pool, const int32_t* init_slots,
                                    const int32_t* final_slots, int64_t n_pool, float* o,
                                    int64_t H, int64_t d_k, int64_t d_v, kda_dtype in_dtype,
                                    void* workspace, int64_t workspace_bytes, void* stream)
{
    kda_status st;
    if ((st = check_packed(N, T_total, H, d_k, d_v, in_dtype)) != KDA_OK) return st;
    if (n_pool < 0 || pool_too_big(n_pool, H)) return KDA_ERR_SHAPE;
    if ((st = check_workspace(workspace, workspace_bytes)) != KDA_OK) return st;
    if (N == 0) return KDA_OK;
    if (!cu_seqlens) return KDA_ERR_NULL;
    if (misaligned(cu_seqlens)) return KDA_ERR_ALIGN;
    if ((init_slots || final_slots) && !state_pool) return KDA_ERR_NULL;
    if ((st = check_ptrs({}, {state_pool, init_slots, final_slots})) != KDA_OK) return st;
    if (T_total > 0 && (st = check_ptrs({q, k, v, beta, log_alpha, o}, {})) != KDA_OK) return st;
    if (T_total == 0 && !final_slots) return KDA_OK;
    kda::StateRefs refs;
    refs.init = init_slots ? state_pool : nullptr;
    refs.fin = final_slots ? state_pool : nullptr;
    refs.init_slots = init_slots;
    refs.fin_slots = final_slots;
    refs.n_pool = n_pool;
    return run_prefill(q, k, v, beta, log_alpha, cu_seqlens, N, 0, T_total, H, refs, o, in_dtype,
                       false, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

kda_status kda_decode_step_slots(const void* q, const void* k, const void* v, const void* beta,
                                 const float* log_alpha, float* state_pool, const int32_t* slots,
                                 int64_t n_pool, float* o, int64_t N, int64_t H, int64_t d_k,
                                 int64_t d_v, kda_dtype in_dtype, void* stream)
{
    kda_status st;
    if ((st = check_dtype(in_dtype)) != KDA_OK) return st;
    if ((st = check_dims(H, d_k, d_v)) != KDA_OK) return st;
    if (N < 0 || n_pool < 0) return KDA_ERR_SHAPE;
    if (N > int64_t(1) << 24 || N * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (pool_too_big(n_pool, H)) return KDA_ERR_SHAPE;
    if (N == 0) return KDA_OK;
    if ((st = check_ptrs({q, k, v, beta, log_alpha, state_pool, slots, o}, {})) != KDA_OK) return st;
    if ((st = no_pending_error()) != KDA_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = debug_check(log_alpha, N * H * kda::kDim, false, nullptr, 0, 0, s)) != KDA_OK) return st;
    return from_hip(kda::launch_decode_step(q, k, v, beta, log_alpha, state_pool, slots, n_pool, o,
                                            N * H, H, in_dtype == KDA_BF16, false, s));
}

kda_status kda_decode_tokens(const void* q, const void* k, const void* v, const void* beta,
                             const float* log_alpha, float* state, const int32_t* n_commit, float* o,
                             int64_t N, int64_t K, int64_t H, int64_t d_k, int64_t d_v,
                             kda_dtype in_dtype, void* stream)
{
    kda_status st;
    if ((st = check_dtype(in_dtype)) != KDA_OK) return st;
    if ((st = check_dims(H, d_k, d_v)) != KDA_OK) return st;
    if (N < 0 || K < 1 || K > kda::kMaxDraft) return KDA_ERR_SHAPE;
    if (N > int64_t(1) << 24 || N * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (N == 0) return KDA_OK;
    if ((st = check_ptrs({q, k, v, beta, log_alpha, state, o}, {n_commit})) != KDA_OK) return st;
    if ((st = no_pending_error()) != KDA_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = debug_check(log_alpha, N * K * H * kda::kDim, false, nullptr, 0, 0, s)) != KDA_OK)
        return st;
    return from_hip(kda::launch_decode_tokens(q, k, v, beta, log_alpha, state, n_commit, o, N, K, H,
                                              in_dtype == KDA_BF16, s));
}

kda_status kda_backward(const void* q, const void* k, const void* v, const void* beta,
                        const float* log_alpha, const float* initial_state, const float* d_o,
                        const float* d_final_state, float* dq, float* dk, float* dv, float* dbeta,
                        float* dlog_alpha, float* d_initial_state, int64_t B, int64_t T, int64_t H,
                        int64_t d_k, int64_t d_v, kda_dtype in_dtype, void* workspace,
                        int64_t workspace_bytes, void* stream)
{
    return backward_impl(q, k, v, beta, log_alpha, nullptr, B, T, 0, initial_state, d_o,
                         d_final_state, dq, dk, dv, dbeta, dlog_alpha, d_initial_state, H, d_k,
                         d_v, in_dtype, workspace, workspace_bytes, stream);
}

kda_status kda_varlen_backward(const void* q, const void* k, const void* v, const void* beta,
                               const float* log_alpha, const int32_t* cu_seqlens, int64_t N,
                               int64_t T_total, const float* initial_state, const float* d_o,
                               const float* d_final_state, float* dq, float* dk, float* dv,
                               float* dbeta, float* dlog_alpha, float* d_initial_state, int64_t H,
                               int64_t d_k, int64_t d_v, kda_dtype in_dtype, void* workspace,
                               int64_t workspace_bytes, void* stream)
{
    if (N > 0 && !cu_seqlens) return KDA_ERR_NULL;
    return backward_impl(q, k, v, beta, log_alpha, cu_seqlens, N, 0, T_total, initial_state, d_o,
                         d_final_state, dq, dk, dv, dbeta, dlog_alpha, d_initial_state, H, d_k,
                         d_v, in_dtype, workspace, workspace_bytes, stream);
}

kda_status kda_prefill_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                                      kda_dtype in_dtype, kda_plan plan, int64_t* bytes)
{
    return prefill_size(false, B, T, 0, H, d_k, d_v, in_dtype, plan, bytes);
}

kda_status kda_varlen_prefill_workspace_size(int64_t N, int64_t T_total, int64_t H, int64_t d_k,
                                             int64_t d_v, kda_dtype in_dtype, kda_plan plan,
                                             int64_t* bytes)
{
    return prefill_size(true, N, 0, T_total, H, d_k, d_v, in_dtype, plan, bytes);
}

kda_status kda_backward_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                                       kda_dtype in_dtype, int64_t* bytes)
{
    return backward_size(false, B, T, 0, H, d_k, d_v, in_dtype, bytes);
}

kda_status kda_varlen_backward_workspace_size(int64_t N, int64_t T_total, int64_t H, int64_t d_k,
                                              int64_t d_v, kda_dtype in_dtype, int64_t* bytes)
{
    return backward_size(true, N, 0, T_total, H, d_k, d_v, in_dtype, bytes);
}

kda_status kda_set_prefill_segment(int64_t tokens)
{
    if (tokens < 0 || tokens % 64 != 0 || tokens > (int64_t(1) << 40)) return KDA_ERR_SHAPE;
    kda::set_forced_segment(tokens);
    return KDA_OK;
}

const char* kda_status_str(kda_status status)
{
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: a size is negative, zero where it may not be, or too large";
        case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unknown input dtype";
        case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: a pointer is not 16-byte aligned (a workspace: 256-byte)";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: only d_k = d_v = 128 is supported";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime rejected a launch, or an earlier HIP error is pending";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: the workspace is too small, or the library could not allocate one";
        case KDA_ERR_PRECONDITION: return "KDA_ERR_PRECONDITION: (KDA_DEBUG) log_alpha not finite or > 0, or cu_seqlens not 0..T_total non-decreasing";
        case KDA_ERR_OVERLAP: return "KDA_ERR_OVERLAP: an output buffer overlaps an input or another output";
    }
    return "KDA_ERR_UNKNOWN: not a kda_status value";
}

int kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
