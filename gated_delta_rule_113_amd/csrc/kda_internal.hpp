// Host-side launchers of the KDA kernels (implemented next to each kernel).
// Sizes have been validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kDim = 128;  // d_k = d_v handled by the kernels
constexpr int64_t kMaxHeads = 65536;  // keeps in-chunk element offsets within 32 bits

// One fused decode step for `units` = N * H heads.
hipError_t launch_decode_step(const void* q, const void* k, const void* v, const void* beta,
                              const float* log_alpha, float* state, float* o, int64_t units,
                              bool bf16, hipStream_t stream);

// Token-by-token prefill with the state held in registers.  Dense when
// cu_seqlens == nullptr (sequence n = rows n*T .. n*T+T-1), packed otherwise.
hipError_t launch_prefill_recurrent(const void* q, const void* k, const void* v,
                                    const void* beta, const float* log_alpha,
                                    const int32_t* cu_seqlens, int64_t n_seq, int64_t T,
                                    int64_t H, const float* initial_state, float* o,
                                    float* final_state, bool bf16, hipStream_t stream);

// Chunked prefill on bf16 matrix instructions (bf16 inputs only): 64-token
// chunks, one workgroup per (sequence, head, segment).  Long sequences are cut
// into segments whose affine state maps are composed in between (three
// launches plus a workspace from a stream-ordered pool); short ones take one
// launch.  Dense when cu_seqlens == nullptr (T rows each), packed otherwise
// (T_total rows in all).
hipError_t launch_prefill_scan(const void* q, const void* k, const void* v, const void* beta,
                               const float* log_alpha, const int32_t* cu_seqlens, int64_t n_seq,
                               int64_t T, int64_t T_total, int64_t H,
                               const float* initial_state, float* o, float* final_state,
                               hipStream_t stream);

// Tokens per segment for the chunked prefill (a positive multiple of 64), or
// 0 to choose it from the problem size and the number of CUs.
void set_prefill_segment(int64_t tokens);

}  // namespace kda
