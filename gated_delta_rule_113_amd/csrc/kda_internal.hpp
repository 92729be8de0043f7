// Host-side launchers of the KDA kernels (implemented next to each kernel).
// Sizes have been validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kDim = 128;  // d_k = d_v handled by the kernels
constexpr int64_t kMaxHeads = 65536;  // keeps in-chunk element offsets within 32 bits
constexpr int64_t kChunk = 64;        // tokens per chunk of the chunked kernels
constexpr int64_t kStateFloats = int64_t(kDim) * kDim;

// Where the entering and leaving states of the sequences live.  Without slot
// arrays, sequence n uses entry n of `init` / `fin` ([*, H, 128, 128] fp32).
// With a slot array, sequence n uses entry slots[n] of a pool of n_pool
// entries, and a slot outside [0, n_pool) means "none": zeros coming in,
// nothing written going out.  A NULL `init` means zeros for every sequence, a
// NULL `fin` that no state is written.
struct StateRefs {
    const float* init = nullptr;
    float* fin = nullptr;
    const int32_t* init_slots = nullptr;
    const int32_t* fin_slots = nullptr;
    int64_t n_pool = 0;
};

// One fused decode step for `units` = N * H heads.  Sequence n's state is
// entry n of `state`, or with `slots` entry slots[n] of a pool of n_pool
// entries (a slot outside [0, n_pool) skips the sequence).
// With `raw`, q and k are unnormalised, beta holds logits and log_alpha gate
// logits (the *_raw entry points of kda.h).
hipError_t launch_decode_step(const void* q, const void* k, const void* v, const void* beta,
                              const float* log_alpha, float* state, const int32_t* slots,
                              int64_t n_pool, float* o, int64_t units, int64_t H, bool bf16,
                              bool raw, hipStream_t stream);

// K (<= kMaxDraft) consecutive tokens of each of N sequences from its state
// (inputs [N, K, H, *], outputs [N, K, H, 128]); with n_commit the state is
// overwritten in place by the state after the first n_commit[n] tokens.
constexpr int64_t kMaxDraft = 16;
hipError_t launch_decode_tokens(const void* q, const void* k, const void* v, const void* beta,
                                const float* log_alpha, float* state, const int32_t* n_commit,
                                float* o, int64_t N, int64_t K, int64_t H, bool bf16,
                                hipStream_t stream);

// Token-by-token prefill with the state held in registers.  Dense when
// cu_seqlens == nullptr (sequence n = rows n*T .. n*T+T-1), packed otherwise.
// With max_len > 0, sequences longer than max_len are skipped (left to the
// chunked kernel).
hipError_t launch_prefill_recurrent(const void* q, const void* k, const void* v,
                                    const void* beta, const float* log_alpha,
                                    const int32_t* cu_seqlens, int64_t n_seq, int64_t T,
                                    int64_t H, const StateRefs& st, float* o, bool bf16,
                                    bool raw, int64_t max_len, hipStream_t stream);

// bf16 sequences of at most this many tokens take the token-by-token kernel:
// below it the chunked kernel's fixed cost per (sequence, head) dominates.
constexpr int64_t kShortPrefill = 16;

// Chunked prefill on bf16 matrix instructions (bf16 inputs only): 64-token
// chunks, one workgroup per (sequence, head, segment).  Long sequences are cut
// into segments whose affine state maps are composed in between (three
// launches plus a workspace); short ones take one launch.  Dense when
// cu_seqlens == nullptr (T rows each), packed otherwise (T_total rows in all).
// With short_max > 0, sequences of at most short_max tokens are skipped (left
// to the token-by-token kernel); short_max <= 64.
//
// A plan fixes the segmentation and the workspace it needs.  Tier 0 is the
// fastest plan: segments, with the split T and P of every mapped chunk kept
// for pass 3 while those images stay under a cap; tier 1 the same segments
// without the images; tier 2 one workgroup per (sequence, head) and no
// workspace.  A tier that would not cut any sequence comes back as tier 2.
// The plans are host arithmetic only (kda_plan.cpp).
constexpr int64_t kMinSegment = 1024;   // shortest automatic segment
constexpr size_t kTpBytes = 4 * 336 * 16;   // the kept chunks of the split T and P of one chunk (T hi, T lo, P hi, P lo)
// The fastest plan keeps the T/P images only while one call needs at most
// this many bytes of them: the million-token workload (32 heads) would need
// 17 GB of them for about 1% less time.
constexpr double kTpCap = static_cast<double>(int64_t(8) << 30);
struct PrefillPlan {
    int tier = 2;
    bool segmented = false;
    bool tp = false;            // pass 1 keeps T and P for pass 3
    int64_t seg = 0;            // tokens per segment (packed: the longest candidate)
    int64_t seg0 = 0;           // dense: tokens of the first segment
    int64_t seg_min = 0;        // packed: the shortest candidate length
    int64_t nseg_dense = 0;     // dense: segments per sequence
    int64_t n_segs = 0;         // segment slots of the grid
    int64_t slots = 0;          // workspace slots (maps and entering states)
    int64_t tp_blocks = 0;      // T/P images per head
    size_t plan_bytes = 0;      // packed: the plan kernel's tables
    size_t ws_bytes = 0;        // workspace bytes in all
};
PrefillPlan plan_prefill_scan(bool packed, int64_t n_seq, int64_t T, int64_t T_total, int64_t H,
                              int n_cu, int64_t forced_segment, int tier);
// ws: at least plan.ws_bytes bytes of device memory, 256-byte aligned (unused
// when the plan is not segmented).  n_cu: compute units the plan was made for.
hipError_t launch_prefill_scan(const void* q, const void* k, const void* v, const void* beta,
                               const float* log_alpha, const int32_t* cu_seqlens, int64_t n_seq,
                               int64_t T, int64_t H, const StateRefs& st, float* o, bool raw,
                               int64_t short_max, const PrefillPlan& plan, void* ws, int n_cu,
                               hipStream_t stream);

// Backward pass (gradients in q, k, v, beta, log_alpha and the initial state
// from those in o and the final state); dense or packed as the prefill.
// Gradients are fp32 in the layouts of their inputs.  bf16 inputs take the
// chunked form (kda_backward_chunk.hip), whose workspace holds
// kChunkBackwardFloats per (chunk id, head).  fp32 inputs take the
// token-by-token chain rule (kda_backward.hip): its forward sweep stores a
// checkpoint state every kBackwardBlock tokens (8 KiB per head-token) in the
// workspace, and the reverse sweep recomputes each block from its checkpoint.
constexpr int kBackwardBlock = 8;
// per (chunk, head): entering state, leaving-state gradient, A / P / T
constexpr size_t kChunkBackwardFloats = 2 * kStateFloats + 3 * kChunk * kChunk;
struct BackwardPlan {
    bool chunked = false;       // bf16 inputs: the chunked matrix-core backward
    int64_t n_ids = 0;          // chunked: chunk ids per head
    int64_t n_slots = 0;        // token-by-token: checkpoint slots per head
    size_t ws_bytes = 0;        // workspace bytes in all
};
BackwardPlan plan_backward(bool packed, int64_t n_seq, int64_t T, int64_t T_total, int64_t H,
                          bool bf16);
hipError_t launch_backward_chunked(const void* q, const void* k, const void* v, const void* beta,
                                   const float* log_alpha, const float* d_o, const int32_t* cu_seqlens,
                                   int64_t n_seq, int64_t T, int64_t H, const float* initial_state,
                                   const float* d_final_state, float* dq, float* dk, float* dv,
                                   float* dbeta, float* dlog_alpha, float* d_initial_state,
                                   int64_t n_ids, void* ws, hipStream_t stream);
// ws: at least plan.ws_bytes bytes of device memory, 256-byte aligned.
// bf16 must match the plan (chunked); fp32 inputs take the token-by-token path.
hipError_t launch_backward(const void* q, const void* k, const void* v, const void* beta,
                           const float* log_alpha, const float* d_o, const int32_t* cu_seqlens,
                           int64_t n_seq, int64_t T, int64_t H, const float* initial_state,
                           const float* d_final_state, float* dq, float* dk, float* dv,
                           float* dbeta, float* dlog_alpha, float* d_initial_state, bool bf16,
                           const BackwardPlan& plan, void* ws, hipStream_t stream);

// ---- runtime helpers (kda_runtime.cpp)

// Compute units of a device (cached; 256 if the query fails).
int cu_count(int dev);

// The opt-in workspace of a call made with KDA_WORKSPACE_AUTO: taken in
// stream order from a per-device pool whose release threshold is 0 (freed
// blocks go back to the device at the next synchronisation) and returned in
// stream order by release().
struct StreamWorkspace {
    void* ptr = nullptr;
    hipStream_t stream = nullptr;
    hipError_t acquire(size_t bytes, hipStream_t s);
    hipError_t release();
    ~StreamWorkspace() { (void)release(); }
};

// With KDA_DEBUG set in the environment, failed HIP calls are printed to stderr.
void report(const char* what, hipError_t e);
bool debug_enabled();

// The scratch of kda_prefill_noalloc (kda_noalloc.hip): a file-scope device
// array of this many bytes per device; *ptr receives its address on the
// current device (looked up once per device).
// 160 MiB holds the segments plan of every dense prefill at the automatic
// segment length on 256 compute units (at most about 144 MiB: fewer than
// 3 x 256 segment slots of 192 KiB).
constexpr size_t kNoallocScratchBytes = size_t(160) << 20;
hipError_t noalloc_scratch(void** ptr);

// KDA_DEBUG precondition checks (kda_checks.hip): the bits of *violations
// name what failed.  The gates are n_gates floats (log alpha <= 0 and finite,
// or with raw only finite); cu_seqlens, if given, n_seq + 1 offsets.  Enqueues
// on `stream` and synchronises it.
constexpr unsigned int kViolationGate = 1u, kViolationStart = 2u, kViolationOrder = 4u,
                       kViolationEnd = 8u;
hipError_t check_preconditions(const float* log_alpha, int64_t n_gates, bool raw,
                               const int32_t* cu_seqlens, int64_t n_seq, int64_t T_total,
                               hipStream_t stream, unsigned int* violations);

// Tokens per segment forced by kda_set_prefill_segment (0 = automatic).
int64_t forced_segment();
void set_forced_segment(int64_t tokens);


}  // namespace kda
