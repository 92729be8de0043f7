// C ABI of libkda.so (declared in include/kda.h): host-side validation, then
// asynchronous launches on the caller's stream.  Nothing here synchronises or
// touches device memory (the segmented prefill's workspace is taken and
// returned in stream order by its launcher); every check happens before a
// launch so that on error nothing is enqueued.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

#include "kda_internal.hpp"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 46;  // keeps every index product in int64

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

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

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// bf16 inputs take the chunked matrix-core kernel, except sequences of at most
// kShortPrefill tokens; fp32 inputs (whose q and k are not exact in bf16) and
// those short sequences take the register-resident token-by-token kernel.
hipError_t launch_prefill(const void* q, const void* k, const void* v, const void* beta,
                          const float* log_alpha, const int32_t* cu_seqlens, int64_t n_seq,
                          int64_t T, int64_t T_total, int64_t H, const kda::StateRefs& st,
                          float* o, kda_dtype in_dtype, bool raw, hipStream_t stream)
{
    if (in_dtype != KDA_BF16)
        return kda::launch_prefill_recurrent(q, k, v, beta, log_alpha, cu_seqlens, n_seq, T, H,
                                             st, o, false, raw, 0, stream);
    // bf16: short sequences token by token, the others chunked.  Each kernel
    // skips the other's sequences (packed lengths are known on the device only).
    const int64_t longest = cu_seqlens ? T_total : T;
    if (longest <= kda::kShortPrefill)
        return kda::launch_prefill_recurrent(q, k, v, beta, log_alpha, cu_seqlens, n_seq, T, H,
                                             st, o, true, raw, 0, stream);
    const hipError_t e = kda::launch_prefill_scan(q, k, v, beta, log_alpha, cu_seqlens, n_seq, T,
                                                  T_total, H, st, o, raw,
                                                  cu_seqlens ? kda::kShortPrefill : 0, stream);
    if (e != hipSuccess || !cu_seqlens) return e;
    return kda::launch_prefill_recurrent(q, k, v, beta, log_alpha, cu_seqlens, n_seq, T, H, st,
                                         o, true, raw, kda::kShortPrefill, stream);
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

kda_status prefill_impl(const void* q, const void* k, const void* v, const void* beta,
                       const float* log_alpha, const float* initial_state, float* o,
                       float* final_state, int64_t B, int64_t T, int64_t H, int64_t d_k,
                       int64_t d_v, kda_dtype in_dtype, bool raw, void* stream)
{
    kda_status st;
    if ((st = check_dtype(in_dtype)) != KDA_OK) return st;
    if ((st = check_dims(H, d_k, d_v)) != KDA_OK) return st;
    if (B < 0 || T < 0) return KDA_ERR_SHAPE;
    if (B > 0 && T > kMaxElems / B) return KDA_ERR_SHAPE;
    if ((st = check_rows(B * T, H)) != KDA_OK) return st;
    if (B > int64_t(1) << 24 || B * H > int64_t(1) << 30) return KDA_ERR_SHAPE;
    if (B == 0) return KDA_OK;
    if (T > 0) {
        if ((st = check_ptrs({q, k, v, beta, log_alpha, o}, {initial_state, final_state})) != KDA_OK)
            return st;
    } else if ((st = check_ptrs({}, {initial_state, final_state})) != KDA_OK) {
        return st;
    }
    if (T == 0 && !final_state) return KDA_OK;
    return from_hip(launch_prefill(q, k, v, beta, log_alpha, nullptr, B, T, B * T, H,
                                   plain_states(initial_state, final_state), o, in_dtype, raw,
                                   static_cast<hipStream_t>(stream)));
}

kda_status varlen_impl(const void* q, const void* k, const void* v, const void* beta,
                              const float* log_alpha, const int32_t* cu_seqlens, int64_t N,
                              int64_t T_total, const float* initial_state, float* o,
                              float* final_state, int64_t H, int64_t d_k, int64_t d_v,
                              kda_dtype in_dtype, bool raw, void* stream)
{
    kda_status st;
    if ((st = check_dtype(in_dtype)) != KDA_OK) return st;
    if ((st = check_dims(H, d_k, d_v)) != KDA_OK) return st;
    if (N < 0 || T_total < 0) return KDA_ERR_SHAPE;
    // cu_seqlens holds int32 row indices
    if (T_total > INT32_MAX || N > int64_t(1) << 24 || N * H > int64_t(1) << 30) return KDA_ERR_SHAPE;
    if ((st = check_rows(T_total, H)) != KDA_OK) return st;
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
    return from_hip(launch_prefill(q, k, v, beta, log_alpha, cu_seqlens, N, 0, T_total, H,
                                   plain_states(initial_state, final_state), o, in_dtype, raw,
                                   static_cast<hipStream_t>(stream)));
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
    return from_hip(kda::launch_decode_step(q, k, v, beta, log_alpha, state, nullptr, 0, o, N * H,
                                            H, in_dtype == KDA_BF16, raw,
                                            static_cast<hipStream_t>(stream)));
}

kda_status backward_impl(const void* q, const void* k, const void* v, const void* beta,
                         const float* log_alpha, const int32_t* cu_seqlens, int64_t n_seq,
                         int64_t T, int64_t T_total, const float* initial_state, const float* d_o,
                         const float* d_final_state, float* dq, float* dk, float* dv, float* dbeta,
                         float* dlog_alpha, float* d_initial_state, int64_t H, int64_t d_k,
                         int64_t d_v, kda_dtype in_dtype, void* stream)
{
    kda_status st;
    if ((st = check_dtype(in_dtype)) != KDA_OK) return st;
    if ((st = check_dims(H, d_k, d_v)) != KDA_OK) return st;
    if (n_seq < 0 || T < 0 || T_total < 0) return KDA_ERR_SHAPE;
    if (cu_seqlens && T_total > INT32_MAX) return KDA_ERR_SHAPE;
    if (!cu_seqlens && n_seq > 0 && T > kMaxElems / n_seq) return KDA_ERR_SHAPE;
    const int64_t rows = cu_seqlens ? T_total : n_seq * T;
    if ((st = check_rows(rows, H)) != KDA_OK) return st;
    if (n_seq > int64_t(1) << 24 || n_seq * H > int64_t(1) << 30) return KDA_ERR_SHAPE;
    if (n_seq == 0) return KDA_OK;
    if (cu_seqlens && misaligned(cu_seqlens)) return KDA_ERR_ALIGN;
    if (rows > 0) {
        if ((st = check_ptrs({q, k, v, beta, log_alpha, d_o, dq, dk, dv, dbeta, dlog_alpha},
                             {initial_state, d_final_state, d_initial_state})) != KDA_OK)
            return st;
    } else if ((st = check_ptrs({}, {initial_state, d_final_state, d_initial_state})) != KDA_OK) {
        return st;
    }
    if (rows == 0 && !d_initial_state) return KDA_OK;
    return from_hip(kda::launch_backward(q, k, v, beta, log_alpha, d_o, cu_seqlens, n_seq, T,
                                         T_total, H, initial_state, d_final_state, dq, dk, dv,
                                         dbeta, dlog_alpha, d_initial_state, in_dtype == KDA_BF16,
                                         static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

kda_status kda_prefill(const void* q, const void* k, const void* v, const void* beta,
                       const float* log_alpha, const float* initial_state, float* o,
                       float* final_state, int64_t B, int64_t T, int64_t H, int64_t d_k,
                       int64_t d_v, kda_dtype in_dtype, void* stream)
{
    return prefill_impl(q, k, v, beta, log_alpha, initial_state, o, final_state, B, T, H, d_k, d_v,
                        in_dtype, false, stream);
}

kda_status kda_prefill_raw(const void* q, const void* k, const void* v, const void* beta,
                           const float* log_alpha, const float* initial_state, float* o,
                           float* final_state, int64_t B, int64_t T, int64_t H, int64_t d_k,
                           int64_t d_v, kda_dtype in_dtype, void* stream)
{
    return prefill_impl(q, k, v, beta, log_alpha, initial_state, o, final_state, B, T, H, d_k, d_v,
                        in_dtype, true, stream);
}

kda_status kda_varlen_prefill(const void* q, const void* k, const void* v, const void* beta,
                              const float* log_alpha, const int32_t* cu_seqlens, int64_t N,
                              int64_t T_total, const float* initial_state, float* o,
                              float* final_state, int64_t H, int64_t d_k, int64_t d_v,
                              kda_dtype in_dtype, void* stream)
{
    return varlen_impl(q, k, v, beta, log_alpha, cu_seqlens, N, T_total, initial_state, o,
                       final_state, H, d_k, d_v, in_dtype, false, stream);
}

kda_status kda_varlen_prefill_raw(const void* q, const void* k, const void* v, const void* beta,
                                  const float* log_alpha, const int32_t* cu_seqlens, int64_t N,
                                  int64_t T_total, const float* initial_state, float* o,
                                  float* final_state, int64_t H, int64_t d_k, int64_t d_v,
                                  kda_dtype in_dtype, void* stream)
{
    return varlen_impl(q, k, v, beta, log_alpha, cu_seqlens, N, T_total, initial_state, o,
                       final_state, H, d_k, d_v, in_dtype, true, stream);
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
                                    void* stream)
{
    kda_status st;
    if ((st = check_dtype(in_dtype)) != KDA_OK) return st;
    if ((st = check_dims(H, d_k, d_v)) != KDA_OK) return st;
    if (N < 0 || T_total < 0 || n_pool < 0) return KDA_ERR_SHAPE;
    if (T_total > INT32_MAX || N > int64_t(1) << 24 || N * H > int64_t(1) << 30) return KDA_ERR_SHAPE;
    if ((st = check_rows(T_total, H)) != KDA_OK) return st;
    if (pool_too_big(n_pool, H)) return KDA_ERR_SHAPE;
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
    return from_hip(launch_prefill(q, k, v, beta, log_alpha, cu_seqlens, N, 0, T_total, H, refs,
                                   o, in_dtype, false, static_cast<hipStream_t>(stream)));
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
    return from_hip(kda::launch_decode_step(q, k, v, beta, log_alpha, state_pool, slots, n_pool, o,
                                            N * H, H, in_dtype == KDA_BF16, false,
                                            static_cast<hipStream_t>(stream)));
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
    return from_hip(kda::launch_decode_tokens(q, k, v, beta, log_alpha, state, n_commit, o, N, K, H,
                                              in_dtype == KDA_BF16,
                                              static_cast<hipStream_t>(stream)));
}

kda_status kda_backward(const void* q, const void* k, const void* v, const void* beta,
                        const float* log_alpha, const float* initial_state, const float* d_o,
                        const float* d_final_state, float* dq, float* dk, float* dv, float* dbeta,
                        float* dlog_alpha, float* d_initial_state, int64_t B, int64_t T, int64_t H,
                        int64_t d_k, int64_t d_v, kda_dtype in_dtype, void* stream)
{
    return backward_impl(q, k, v, beta, log_alpha, nullptr, B, T, 0, initial_state, d_o,
                         d_final_state, dq, dk, dv, dbeta, dlog_alpha, d_initial_state, H, d_k,
                         d_v, in_dtype, stream);
}

kda_status kda_varlen_backward(const void* q, const void* k, const void* v, const void* beta,
                               const float* log_alpha, const int32_t* cu_seqlens, int64_t N,
                               int64_t T_total, const float* initial_state, const float* d_o,
                               const float* d_final_state, float* dq, float* dk, float* dv,
                               float* dbeta, float* dlog_alpha, float* d_initial_state, int64_t H,
                               int64_t d_k, int64_t d_v, kda_dtype in_dtype, void* stream)
{
    if (N > 0 && !cu_seqlens) return KDA_ERR_NULL;
    return backward_impl(q, k, v, beta, log_alpha, cu_seqlens, N, 0, T_total, initial_state, d_o,
                         d_final_state, dq, dk, dv, dbeta, dlog_alpha, d_initial_state, H, d_k,
                         d_v, in_dtype, stream);
}

kda_status kda_set_prefill_segment(int64_t tokens)
{
    if (tokens < 0 || tokens % 64 != 0 || tokens > (int64_t(1) << 40)) return KDA_ERR_SHAPE;
    kda::set_prefill_segment(tokens);
    return KDA_OK;
}

kda_status kda_set_prefill_tp_limit(int64_t bytes)
{
    if (bytes < 0) return KDA_ERR_SHAPE;
    kda::set_prefill_tp_limit(bytes);
    return KDA_OK;
}

const char* kda_status_str(kda_status status)
{
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: a size is negative, zero where it may not be, or too large";
        case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unknown input dtype";
        case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: a pointer is not 16-byte aligned";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: only d_k = d_v = 128 is supported";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime rejected a launch";
    }
    return "KDA_ERR_UNKNOWN: not a kda_status value";
}

int kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
