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
 *    the caller.  The library keeps no device memory between calls.
 *  - Workspace.  The prefill calls on bf16 inputs cut long sequences into
 *    segments (see kda_set_prefill_segment) and need device scratch memory
 *    for the segment maps; the backward calls need it for their state
 *    checkpoints.  Those calls take two arguments for it:
 *      workspace, workspace_bytes : caller-owned device memory, 256-byte
 *          aligned (KDA_ERR_ALIGN), of workspace_bytes bytes (NULL when 0).
 *          It is used in stream order: it must stay allocated and must not be
 *          used for anything else until the call's work on `stream` is done.
 *          Its contents on entry do not matter and are undefined afterwards.
 *      workspace_bytes = KDA_WORKSPACE_AUTO (workspace NULL) : the library
 *          takes the workspace itself, in stream order on `stream`, from a
 *          per-device pool whose release threshold is 0 (freed memory goes
 *          back to the device at the next synchronisation, nothing stays
 *          reserved), and returns it in stream order at the end of the call.
 *          If that allocation fails the call returns KDA_ERR_WORKSPACE and
 *          enqueues nothing.
 *    The *_workspace_size calls below give the bytes of each plan.  A prefill
 *    takes the fastest plan whose workspace fits workspace_bytes: FULL, else
 *    SEGMENTS, else UNSEGMENTED (which needs none, so a prefill always runs;
 *    with little work per compute unit it is much slower).  A backward call
 *    with less than its workspace size returns KDA_ERR_WORKSPACE.
 *  - Calls are re-entrant and thread-safe (the one knob,
 *    kda_set_prefill_segment, is an atomic process-wide setting for tests and
 *    tuning).
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
 *  - Every tensor pointer must be 16-byte aligned (KDA_ERR_ALIGN).
 *  - Preconditions on device data: log_alpha finite and <= 0 (the *_raw
 *    calls: gate logits finite); cu_seqlens[0] = 0, non-decreasing,
 *    cu_seqlens[N] = T_total.  They are not checked unless KDA_DEBUG is set in
 *    the environment: then every call first runs a check kernel and
 *    synchronises `stream` (so it cannot be captured into a graph), and
 *    returns KDA_ERR_PRECONDITION, enqueueing nothing more, on a violation.
 *    KDA_DEBUG also prints failed HIP calls to stderr.
 *  - The calling thread's current device (hipSetDevice) must be the device
 *    that holds the pointers and `stream`: plans and workspace sizes follow
 *    its compute-unit count.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *    asynchronous on it: arguments are validated on the host first, and on any
 *    error nothing is enqueued.  No call synchronises (KDA_DEBUG aside).  A
 *    fault inside a kernel surfaces at the caller's next synchronisation.
 *  - A HIP error left unread by an earlier call of the calling thread is not
 *    cleared: the call enqueues nothing and returns KDA_ERR_HIP, and the error
 *    stays for the caller to read (hipGetLastError).
 *  - Inputs must not overlap outputs, except where stated.
 */
#ifndef KDA_H
#define KDA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 3

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,         /* a required pointer is NULL                    */
    KDA_ERR_SHAPE = 2,        /* a size is negative, zero where it may not be, or too large */
    KDA_ERR_DTYPE = 3,        /* in_dtype is not a kda_dtype value             */
    KDA_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned              */
    KDA_ERR_UNSUPPORTED = 5,  /* d_k or d_v other than 128                      */
    KDA_ERR_HIP = 6,          /* the HIP runtime rejected a launch, or a HIP error is pending */
    KDA_ERR_WORKSPACE = 7,    /* workspace too small or misused, or none could be allocated */
    KDA_ERR_PRECONDITION = 8, /* KDA_DEBUG: a device-data precondition does not hold */
    KDA_ERR_OVERLAP = 9       /* output buffers overlap each other or an input  */
} kda_status;

/* workspace_bytes value asking the library to allocate the workspace itself */
#define KDA_WORKSPACE_AUTO (-1)

/* Prefill plans, fastest first (see the workspace convention above). */
typedef enum kda_plan {
    KDA_PLAN_FULL = 0,        /* segments; pass 1 also keeps the split UT transform
                                 T and query-key matrix P of every chunk it maps
                                 (their lower-triangular parts, 21 KiB per chunk
                                 and head) for pass 3, while those stay under
                                 8 GiB per call */
    KDA_PLAN_SEGMENTS = 1,    /* segments, without the T/P images */
    KDA_PLAN_UNSEGMENTED = 2  /* one workgroup per (sequence, head); no workspace */
} kda_plan;

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
 *   workspace, workspace_bytes : see the workspace convention above
 *                 (kda_prefill_workspace_size gives each plan's bytes)
 * B = 0 is a no-op.  T = 0 writes final_state = initial_state (or zeros).
 * Requires 1 <= H <= 65536.
 */
kda_status kda_prefill(const void *q, const void *k, const void *v, const void *beta,
                       const float *log_alpha, const float *initial_state,
                       float *o, float *final_state,
                       int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                       kda_dtype in_dtype, void *workspace, int64_t workspace_bytes,
                       void *stream);

/*
 * kda_prefill for callers that cannot allocate device memory at all (code
 * under HIP graph capture, serving loops or harnesses that forbid
 * allocation): the same arguments and results as kda_prefill without a
 * workspace argument.  Its workspace is a fixed scratch array of 160 MiB per
 * device inside the library, held from the library's first use of that
 * device until the process ends; the call allocates nothing.
 *   - It takes the fastest plan that fits 160 MiB (see kda_plan).  At the
 *     automatic segment length the KDA_PLAN_SEGMENTS workspace of a dense
 *     prefill on an MI355X (256 compute units) is at most about 144 MiB, so
 *     every such call runs segmented.  A problem whose KDA_PLAN_SEGMENTS
 *     workspace exceeds 160 MiB (only possible with a short length forced by
 *     kda_set_prefill_segment) is refused with KDA_ERR_WORKSPACE and nothing
 *     enqueued, rather than run unsegmented.
 *   - Every call on one device shares that device's scratch, which keeps the
 *     last call's contents (nothing in it needs clearing): calls that overlap
 *     on one device (concurrent streams, or threads) race and give wrong
 *     results.  Serialise them, e.g. on one stream.
 */
kda_status kda_prefill_noalloc(const void *q, const void *k, const void *v, const void *beta,
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
 *   workspace, workspace_bytes : see the workspace convention above
 *                 (kda_varlen_prefill_workspace_size gives each plan's bytes)
 * N = 0 is a no-op.  T_total may be 0 (then every sequence is empty).
 */
kda_status kda_varlen_prefill(const void *q, const void *k, const void *v, const void *beta,
                              const float *log_alpha, const int32_t *cu_seqlens,
                              int64_t N, int64_t T_total,
                              const float *initial_state, float *o, float *final_state,
                              int64_t H, int64_t d_k, int64_t d_v,
                              kda_dtype in_dtype, void *workspace, int64_t workspace_bytes,
                              void *stream);

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
                           kda_dtype in_dtype, void *workspace, int64_t workspace_bytes,
                           void *stream);
kda_status kda_varlen_prefill_raw(const void *q, const void *k, const void *v, const void *beta,
                                  const float *log_alpha, const int32_t *cu_seqlens,
                                  int64_t N, int64_t T_total,
                                  const float *initial_state, float *o, float *final_state,
                                  int64_t H, int64_t d_k, int64_t d_v,
                                  kda_dtype in_dtype, void *workspace, int64_t workspace_bytes,
                                  void *stream);
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
 * 4-Bit and Speculative Decoding"); the per-token update is the decode step's
 * (a verify of K <= 4 tokens evaluates the same recurrence as one block, equal
 * to it up to fp32 rounding).
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
 * state_pool may be NULL only when both slot arrays are NULL.  The workspace
 * is that of kda_varlen_prefill (same sizes, same plans).
 */
kda_status kda_varlen_prefill_slots(const void *q, const void *k, const void *v, const void *beta,
                                    const float *log_alpha, const int32_t *cu_seqlens, int64_t N,
                                    int64_t T_total, float *state_pool, const int32_t *init_slots,
                                    const int32_t *final_slots, int64_t n_pool, float *o,
                                    int64_t H, int64_t d_k, int64_t d_v, kda_dtype in_dtype,
                                    void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Backward pass: the gradients of a loss in the inputs of a prefill, given its
 * gradients in the outputs, for training a KDA layer.  The pages describe the
 * model's training (quantization-aware from fine-tuning onward: "Kimi K3 --
 * the architecture and infrastructure, explained", section "Training
 * infrastructure: quantization-aware from SFT onward"); the gradients are the
 * chain rule taken through the recurrence above.
 * Inputs are those of the prefill call they differentiate:
 *   q, k, v, beta, log_alpha, initial_state : as kda_prefill (dense, [B, T, H, *])
 *                 or kda_varlen_prefill (packed, [T_total, H, *] with
 *                 cu_seqlens in DEVICE memory); initial_state NULL = zeros
 *   d_o           : fp32, the layout of o: the loss gradient in every output
 *   d_final_state : [B or N, H, d_k, d_v] fp32, the loss gradient in the final
 *                 state, or NULL for zeros
 * Outputs, fp32, all written:
 *   dq, dk, dlog_alpha : the layout of q;  dv : the layout of v;  dbeta : the
 *                 layout of beta.  With bf16 inputs dk and dlog_alpha also
 *                 hold intermediate values of the call before their final
 *                 ones, so no output may overlap an input or another output
 *                 (KDA_ERR_OVERLAP, checked on the host from the sizes)
 *   d_initial_state : [B or N, H, d_k, d_v], or NULL to skip; it MAY be the same
 *                 pointer as d_final_state
 * bf16 inputs take the chunked form on the matrix cores (64-token chunks;
 * operands split into hi + lo bf16 as in the prefill, fp32 accumulation): the
 * workspace keeps, per (64-token chunk, head), the chunk's entering state and
 * the gradient in its leaving state, its UT transform, A and P matrices,
 * 176 KiB, i.e. 2.75 KiB per head-token (2.8 GiB for 8 x 4096 tokens x 32
 * heads, 88 GiB for 1,048,576 tokens x 32 heads).  fp32
 * inputs take the token-by-token chain rule with a state checkpoint every 8
 * tokens (8 KiB per head-token).  kda_backward_workspace_size gives the bytes;
 * a smaller workspace is KDA_ERR_WORKSPACE.  B or N = 0 is a no-op; with no
 * tokens, d_initial_state = d_final_state (or zeros).
 */
kda_status kda_backward(const void *q, const void *k, const void *v, const void *beta,
                        const float *log_alpha, const float *initial_state,
                        const float *d_o, const float *d_final_state,
                        float *dq, float *dk, float *dv, float *dbeta, float *dlog_alpha,
                        float *d_initial_state,
                        int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                        kda_dtype in_dtype, void *workspace, int64_t workspace_bytes,
                        void *stream);
kda_status kda_varlen_backward(const void *q, const void *k, const void *v, const void *beta,
                               const float *log_alpha, const int32_t *cu_seqlens,
                               int64_t N, int64_t T_total, const float *initial_state,
                               const float *d_o, const float *d_final_state,
                               float *dq, float *dk, float *dv, float *dbeta,
                               float *dlog_alpha, float *d_initial_state,
                               int64_t H, int64_t d_k, int64_t d_v,
                               kda_dtype in_dtype, void *workspace, int64_t workspace_bytes,
                               void *stream);

/*
 * Workspace sizes.  *bytes receives the device workspace, in bytes, that the
 * call of the same name with these sizes needs on the calling thread's current
 * device (0 when it needs none): for the prefills under the given plan (a plan
 * that would cut no sequence needs none), for the backward calls in all.  The
 * arguments are validated as the calls validate them (a non-OK status leaves
 * *bytes = 0); nothing is enqueued.  The prefill sizes depend on the current
 * device's compute units (a query that needs them and finds no device returns
 * KDA_ERR_HIP) and on kda_set_prefill_segment; the backward sizes depend on
 * the arguments alone.  The *_raw and *_slots prefills take the sizes of their
 * plain forms.
 */
kda_status kda_prefill_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                                      kda_dtype in_dtype, kda_plan plan, int64_t *bytes);
kda_status kda_varlen_prefill_workspace_size(int64_t N, int64_t T_total, int64_t H, int64_t d_k,
                                             int64_t d_v, kda_dtype in_dtype, kda_plan plan,
                                             int64_t *bytes);
kda_status kda_backward_workspace_size(int64_t B, int64_t T, int64_t H, int64_t d_k, int64_t d_v,
                                       kda_dtype in_dtype, int64_t *bytes);
kda_status kda_varlen_backward_workspace_size(int64_t N, int64_t T_total, int64_t H, int64_t d_k,
                                              int64_t d_v, kda_dtype in_dtype, int64_t *bytes);

/*
 * Tuning and testing knob for the bf16 prefill (process-wide and atomic; a
 * call reads it once, and the workspace sizes above follow it, so change it
 * only between a size query and the call it sizes).  The blockwise prefill
 * runs one workgroup per (sequence, head, segment); a sequence longer than
 * `tokens` is cut into segments of `tokens` tokens (the last one shorter),
 * processed in parallel and stitched together through their affine state maps
 * ("blockwise and context-parallel" in "Kimi K3 -- the architecture and
 * infrastructure, explained", section "Kimi Delta Attention: the load-bearing
 * choice").  0 (the default) picks the length from the problem size and the
 * number of compute units; for dense input the first segment of each sequence
 * runs with its outputs while the other segments build their maps, so a
 * sequence takes one segment more, and the last segment is made shorter
 * (about 3/5 of the others under KDA_PLAN_FULL, else the first is 7/8 as
 * long); for packed input a small planning kernel then chooses, on the device
 * where the sequence lengths are, between that length and the powers of two
 * below it (down to an eighth of it).  tokens must be 0 or a positive multiple
 * of 64, else KDA_ERR_SHAPE.  Results do not depend on it beyond rounding.
 */
kda_status kda_set_prefill_segment(int64_t tokens);

/* Static, human-readable name of a status code (never NULL). */
const char *kda_status_str(kda_status status);

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
