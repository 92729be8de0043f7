/*
 * kda.h -- C ABI of libkda.so: Kimi Delta Attention (KDA) prefill and decode
 * on AMD Instinct MI355X (gfx950).
 *
 * KDA keeps, per head, a fixed-size fp32 memory S of d_k x d_v (rows are the
 * d_k = 128 forgetting channels) and updates it once per token with the delta
 * rule under a channel-wise forgetting gate:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,            alpha_t = exp(log_alpha_t)  (one per channel)
 *
 * Sources, by page title and section:
 *  - "Kimi K3 -- the architecture and infrastructure, explained", section
 *    "How the delta rule actually works": the update S <- S - beta (S k - v) k^T
 *    (printed with S as d_v x d_k; stored here transposed, d_k x d_v).
 *  - same page, section "Kimi Delta Attention: the load-bearing choice": the
 *    gate is per channel; the computation is blockwise so it maps onto matrix
 *    units; decode cost per token is constant.
 *  - same page, section "Serving infrastructure: supernodes and the prefill
 *    cache": a cached prefill state is restored and only the new suffix is
 *    processed (hence the optional initial state and the returned final state).
 *  - "Inside Kimi K3: How Moonshot AI Built the Largest Open-Source Model",
 *    section "Technical Details": 128 forgetting dials per head, beta = writing
 *    strength, alpha = forgetting factor, erase then write.
 * Readings where the pages are silent: the decay is applied before the
 * erase/write; beta is one scalar per (token, head); the read-out uses the
 * updated state; there is no query scaling, and the plain calls normalise
 * nothing (the *_raw calls below prepare raw projections themselves).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers (e.g. torch CUDA tensors), owned by
 *    the caller.  Decode allocates nothing.  A prefill whose sequences are
 *    long enough to be cut into segments (see kda_set_prefill_segment) takes
 *    a temporary workspace, allocated and freed in stream order on `stream`
 *    from a memory pool the library keeps per device (no synchronisation);
 *    if that allocation fails the call runs unsegmented instead.  The
 *    backward calls take their state checkpoints from the same pool.  Calls
 *    are re-entrant and thread-safe.
 *  - Layouts are dense row-major, innermost dimension last:
 *        q, k, log_alpha : [rows, H, d_k]      v, o : [rows, H, d_v]
 *        beta            : [rows, H]
 *        states          : [units, H, d_k, d_v]  (d_v contiguous)
 *    where a "row" is one token position (see each call).
 *  - q, k, v and beta share one storage type, `in_dtype` (KDA_F32 or
 *    KDA_BF16); log_alpha, states and o are always fp32.  The state is fp32
 *    and bf16 inputs are widened exactly.  Arithmetic is fp32, except that
 *    the chunked prefill (bf16 inputs, sequences over 16 tokens) forms its
 *    matrix products on bf16 matrix cores from operands split into a high
 *    and a low bf16 part (about 16 significant bits each), accumulating in
 *    fp32.
 *  - Supported sizes: d_k = d_v = 128 (anything else -> KDA_ERR_UNSUPPORTED);
 *    1 <= H <= 65536 heads (anything else -> KDA_ERR_SHAPE).
 *  - Every pointer must be 16-byte aligned (KDA_ERR_ALIGN).
 *  - Preconditions not checked (device data): log_alpha finite and <= 0;
 *    cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N] = T_total.
 *  - The calling thread's current device (hipSetDevice) must be the device
 *    that holds the pointers and `stream`: the segmented prefill takes its
 *    workspace from that device's pool and sizes its work by its CU count.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *    asynchronous on it: arguments are validated on the host first, and on any
 *    error nothing is enqueued.  No call synchronises.  A fault inside a
 *    kernel surfaces at the caller's next synchronisation.
 *  - Inputs must not overlap outputs, except where stated.
 */
#ifndef KDA_H
#define KDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,         /* a required pointer is NULL                    */
    KDA_ERR_SHAPE = 2,        /* a size is negative, zero where it may not be, or too large */
    KDA_ERR_DTYPE = 3,        /* in_dtype is not a kda_dtype value             */
    KDA_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned              */
    KDA_ERR_UNSUPPORTED = 5,  /* d_k or d_v other than 128                      */
    KDA_ERR_HIP = 6           /* the HIP runtime rejected a launch             */
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/*
 * Dense prefill of B sequences of T tokens each, all H heads.
 *   q, k        : [B, T, H, d_k]  in_dtype
 *   v           : [B, T, H, d_v]  in_dtype
 *   beta        : [B, T, H]       in_dtype   (write strength per token and head)
 *   log_alpha   : [B, T, H, d_k]  fp32       (log forgetting factor per channel)
 *   initial_state : [B, H, d_k, d_v] fp32, or NULL for zeros (a restored
 *                 prefill cache; only the given tokens are processed)
 *   o           : [B, T, H, d_v]  fp32, written
 *   final_state : [B, H, d_k, d_v] fp32, written, or NULL to skip; it MAY be
 *                 the same pointer as initial_state (in-place resume)
 * B = 0 is a no-op.  T = 0 writes final_state = initial_state (or zeros).
 * Requires 1 <= H <= 65536.
 */
kda_status kda_prefill(const void *q, const void *k, const void *v, const void *beta,
                       const float *log_alpha, const float *initial_state,
                       float *o, float *final_state,
                       int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                       kda_dtype in_dtype, void *stream);

/*
 * Packed variable-length prefill of N sequences stored back to back.
 *   q, k, log_alpha : [T_total, H, d_k];  v, o : [T_total, H, d_v];  beta : [T_total, H]
 *   cu_seqlens  : [N + 1] int32, DEVICE memory: sequence n owns token rows
 *                 cu_seqlens[n] .. cu_seqlens[n+1]-1.  Read on the device, so
 *                 the call needs no host synchronisation.
 *   initial_state / final_state : [N, H, d_k, d_v] fp32 as in kda_prefill
 *                 (NULL initial state = zeros for every sequence; the two may
 *                 alias).  No state crosses a sequence boundary; an empty
 *                 sequence returns its initial state.
 * N = 0 is a no-op.  T_total may be 0 (then every sequence is empty).
 */
kda_status kda_varlen_prefill(const void *q, const void *k, const void *v, const void *beta,
                              const float *log_alpha, const int32_t *cu_seqlens,
                              int64_t N, int64_t T_total,
                              const float *initial_state, float *o, float *final_state,
                              int64_t H, int64_t d_k, int64_t d_v,
                              kda_dtype in_dtype, void *stream);

/*
 * One decode step: one new token for each of N sequences, all H heads.
 *   q, k, log_alpha : [N, H, d_k];  v : [N, H, d_v];  beta : [N, H]
 *   state : [N, H, d_k, d_v] fp32, read and updated IN PLACE (S_{t-1} -> S_t)
 *   o     : [N, H, d_v] fp32, written (o_t = S_t^T q_t)
 * Each head's state is read once and written once.  N = 0 is a no-op.
 */
kda_status kda_decode_step(const void *q, const void *k, const void *v, const void *beta,
                           const float *log_alpha, float *state, float *o,
                           int64_t N, int64_t H, int64_t d_k, int64_t d_v,
                           kda_dtype in_dtype, void *stream);

/*
 * Raw-input variants: the same calls, arguments and layouts as kda_prefill,
 * kda_varlen_prefill and kda_decode_step, with the inputs as a layer's
 * projections produce them; the preparation runs inside the kernels, so the
 * prepared inputs never make an extra pass through memory.
 *   q, k      : need not be unit vectors; each (token, head) vector is divided
 *               by its L2 norm (a zero vector stays zero) and, for bf16 inputs,
 *               rounded back to bf16 (nearest, ties to even)
 *   beta      : logits b; the write strength is sigmoid(b) = 1 / (1 + e^-b)
 *   log_alpha : gate logits a; the log forgetting factor is
 *               -softplus(a) = -log(1 + e^a), so alpha = 1 / (1 + e^a)
 * The pages give beta (the writing strength) and alpha (the forgetting
 * factor) as two learned gate parameters of KDA ("Inside Kimi K3: How
 * Moonshot AI Built the Largest Open-Source Model", section "Technical
 * Details") without their parameterisation; sigmoid and minus-softplus are the
 * plainest readings that keep both in (0, 1).  Any finite a is valid.
 */
kda_status kda_prefill_raw(const void *q, const void *k, const void *v, const void *beta,
                           const float *log_alpha, const float *initial_state,
                           float *o, float *final_state,
                           int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                           kda_dtype in_dtype, void *stream);
kda_status kda_varlen_prefill_raw(const void *q, const void *k, const void *v, const void *beta,
                                  const float *log_alpha, const int32_t *cu_seqlens,
                                  int64_t N, int64_t T_total,
                                  const float *initial_state, float *o, float *final_state,
                                  int64_t H, int64_t d_k, int64_t d_v,
                                  kda_dtype in_dtype, void *stream);
kda_status kda_decode_step_raw(const void *q, const void *k, const void *v, const void *beta,
                               const float *log_alpha, float *state, float *o,
                               int64_t N, int64_t H, int64_t d_k, int64_t d_v,
                               kda_dtype in_dtype, void *stream);

/*
 * K consecutive tokens (1 <= K <= 16) of each of N sequences from its current
 * state, for speculative decoding: verify K draft tokens in one pass, then
 * keep the accepted prefix.  The pages describe a draft layer that guesses
 * several tokens which the main model then checks in one pass (the
 * marketersindex.com Kimi K3 article, section "Optimization for Inference:
 * 4-Bit and Speculative Decoding"); the per-token update is the decode step's.
 *   q, k, log_alpha : [N, K, H, d_k];  v : [N, K, H, d_v];  beta : [N, K, H]
 *   o      : [N, K, H, d_v] fp32, written for all K tokens
 *   state  : [N, H, d_k, d_v] fp32.  Without n_commit it is only read (verify).
 *   n_commit : int32 [N] in DEVICE memory, or NULL.  With it, sequence n's
 *            state is replaced IN PLACE by the state after its first
 *            n_commit[n] tokens (values are clamped to [0, K]; 0 leaves it
 *            unchanged).  Rolling back to an accepted prefix is a second call
 *            with the accepted counts: the tokens are recomputed from the
 *            unchanged state, which moves fewer bytes than keeping a state
 *            checkpoint per draft token.
 * Each head's state is read once and written at most once.  N = 0 is a no-op;
 * K outside [1, 16] is KDA_ERR_SHAPE.
 */
kda_status kda_decode_tokens(const void *q, const void *k, const void *v, const void *beta,
                             const float *log_alpha, float *state, const int32_t *n_commit,
                             float *o, int64_t N, int64_t K, int64_t H, int64_t d_k, int64_t d_v,
                             kda_dtype in_dtype, void *stream);

/*
 * State pool addressed by slot (serving: continuous batching and a prefill
 * cache whose states are restored and updated without copies).  The pages
 * describe a cached prefill state that is restored so only the new suffix is
 * prefilled ("Kimi K3 -- the architecture and infrastructure, explained",
 * section "Serving infrastructure: supernodes and the prefill cache"); here the
 * states live in one caller-owned pool and each call names, per sequence, the
 * pool entry to use.
 *   state_pool : [n_pool, H, d_k, d_v] fp32, DEVICE memory, caller-owned.
 *   slots      : int32 [N], DEVICE memory, read on the device.  A slot outside
 *                [0, n_pool) means "no entry" (see each call); such a slot
 *                never causes an access outside the pool.
 * Arithmetic is exactly that of the plain calls: a sequence whose state sits
 * in pool entry s gives the same bits as the plain call given that state.
 */

/*
 * One decode step with the states in a pool: sequence n updates pool entry
 * slots[n] IN PLACE (all H heads) and writes o[n].  A sequence whose slot is
 * outside [0, n_pool) is skipped: its pool entries and its rows of o are left
 * untouched (padding rows of a fixed-size batch).  Non-skipped slots must be
 * distinct (two sequences updating one entry race).
 *   q, k, log_alpha : [N, H, d_k];  v : [N, H, d_v];  beta : [N, H];  o : [N, H, d_v]
 * N = 0 is a no-op.
 */
kda_status kda_decode_step_slots(const void *q, const void *k, const void *v, const void *beta,
                                 const float *log_alpha, float *state_pool, const int32_t *slots,
                                 int64_t n_pool, float *o, int64_t N, int64_t H, int64_t d_k,
                                 int64_t d_v, kda_dtype in_dtype, void *stream);

/*
 * Packed variable-length prefill (as kda_varlen_prefill) with the states in a
 * pool.  Sequence n starts from pool entry init_slots[n] (zeros if that slot is
 * outside [0, n_pool), or for every sequence if init_slots is NULL) and leaves
 * its final state in pool entry final_slots[n] (not written if that slot is
 * outside [0, n_pool), or for every sequence if final_slots is NULL).  A
 * sequence may resume in place (init_slots[n] == final_slots[n]); otherwise no
 * final slot may equal another sequence's initial or final slot.
 * state_pool may be NULL only when both slot arrays are NULL.
 */
kda_status kda_varlen_prefill_slots(const void *q, const void *k, const void *v, const void *beta,
                                    const float *log_alpha, const int32_t *cu_seqlens, int64_t N,
                                    int64_t T_total, float *state_pool, const int32_t *init_slots,
                                    const int32_t *final_slots, int64_t n_pool, float *o,
                                    int64_t H, int64_t d_k, int64_t d_v, kda_dtype in_dtype,
                                    void *stream);

/*
 * Backward pass: the gradients of a loss in the inputs of a prefill, given its
 * gradients in the outputs, for training a KDA layer.  The pages describe the
 * model's training (quantization-aware from fine-tuning onward: "Kimi K3 --
 * the architecture and infrastructure, explained", section "Training
 * infrastructure: quantization-aware from SFT onward"); the gradients are the
 * chain rule taken through the recurrence above, token by token in reverse.
 * Inputs are those of the prefill call they differentiate:
 *   q, k, v, beta, log_alpha, initial_state : as kda_prefill (dense, [B, T, H, *])
 *                 or kda_varlen_prefill (packed, [T_total, H, *] with
 *                 cu_seqlens in DEVICE memory); initial_state NULL = zeros
 *   d_o           : fp32, the layout of o: the loss gradient in every output
 *   d_final_state : [B or N, H, d_k, d_v] fp32, the loss gradient in the final
 *                 state, or NULL for zeros
 * Outputs, fp32, all written:
 *   dq, dk, dlog_alpha : the layout of q;  dv : the layout of v;  dbeta : the
 *                 layout of beta
 *   d_initial_state : [B or N, H, d_k, d_v], or NULL to skip; it MAY be the same
 *                 pointer as d_final_state
 * q, k, v, beta are in_dtype (bf16 inputs widened exactly); arithmetic is fp32.
 * The call recomputes the forward states: it runs the recurrence once storing
 * a state every 8 tokens in a workspace taken in stream order from the
 * device's pool (8 KiB per head-token, e.g. 8 GiB for 8 x 4096 tokens x 32
 * heads), then sweeps back recomputing each block from its stored state.  If
 * that allocation fails the call returns KDA_ERR_HIP and enqueues nothing.  B or N = 0 is a no-op; with no
 * tokens, d_initial_state = d_final_state (or zeros).
 */
kda_status kda_backward(const void *q, const void *k, const void *v, const void *beta,
                        const float *log_alpha, const float *initial_state,
                        const float *d_o, const float *d_final_state,
                        float *dq, float *dk, float *dv, float *dbeta, float *dlog_alpha,
                        float *d_initial_state,
                        int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                        kda_dtype in_dtype, void *stream);
kda_status kda_varlen_backward(const void *q, const void *k, const void *v, const void *beta,
                               const float *log_alpha, const int32_t *cu_seqlens,
                               int64_t N, int64_t T_total, const float *initial_state,
                               const float *d_o, const float *d_final_state,
                               float *dq, float *dk, float *dv, float *dbeta,
                               float *dlog_alpha, float *d_initial_state,
                               int64_t H, int64_t d_k, int64_t d_v,
                               kda_dtype in_dtype, void *stream);

/*
 * Tuning and testing knob for the bf16 prefill (process-wide; set it while no
 * prefill call is running).  The blockwise prefill runs one workgroup per
 * (sequence, head, segment); a sequence longer than `tokens` is cut into
 * segments of `tokens` tokens (the last one shorter), processed in parallel
 * and stitched together through their affine state maps ("blockwise and
 * context-parallel" in "Kimi K3 -- the architecture and infrastructure,
 * explained", section "Kimi Delta Attention: the load-bearing choice").
 * 0 (the default) picks the length from the problem size and the number of
 * compute units; for dense input the first segment of each sequence runs
 * with its outputs while the other segments build their maps, so a sequence
 * takes one segment more, and the last segment is made shorter (about 3/5 of
 * the others with the T/P reuse below, else the first is 7/8 as long); for
 * packed input a small planning kernel then chooses, on
 * the device where the sequence lengths are, between that length and the
 * powers of two below it (down to an eighth of it).  tokens must be 0 or a
 * positive multiple of 64, else KDA_ERR_SHAPE.  Results do not depend on it
 * beyond rounding.
 */
kda_status kda_set_prefill_segment(int64_t tokens);

/*
 * Second knob of the bf16 prefill (process-wide, like the one above).  When
 * a sequence (dense or packed) is cut into segments, pass 1 (which builds the
 * segment maps) also keeps the split UT transform T = (I + Diag(beta) A)^-1
 * and query-key matrix P of every chunk it maps, 32 KiB per chunk and head,
 * and pass 3 reuses them instead of forming them again.  That workspace (one
 * block per 64 rows of the input plus one per sequence, per head) comes from
 * the same stream-ordered pool as the rest and is used only while one call
 * needs at most `bytes` of it (default 8 GiB; 0 turns it off, and for dense
 * input the first segment is then made shorter instead).  If the pool cannot
 * provide it, the call goes without it.  Results do not depend on it beyond
 * rounding.  bytes < 0 is KDA_ERR_SHAPE.
 */
kda_status kda_set_prefill_tp_limit(int64_t bytes);

/* Static, human-readable name of a status code (never NULL). */
const char *kda_status_str(kda_status status);

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
