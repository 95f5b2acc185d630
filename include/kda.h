/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention operator.
 *
 * The operator is the channel-wise gated delta rule of the page
 * "Kimi Delta Attention" (architecture deep dive), §03 "KDA's specific
 * innovation":
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                      (§02, read after the update)
 *
 * with S a dk x dv matrix per (sequence, head).  §06 "From recurrence to GPU
 * kernels" names its two execution modes, which are the two entry points:
 * a chunk-parallel prefill over blocks of tokens that carries only the final
 * state across blocks (kda_prefill_varlen), and a fused recurrent step that
 * consumes one q/k/v and gate set and updates the state in place
 * (kda_decode_step).  §07 "Prefix caching and state transport" fixes the
 * state interface: initial and final recurrent states in, and out of, the
 * prefill, so a prefix state can be restored and continued.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor arguments are DEVICE pointers to contiguous, row-major
 *   buffers, 16-byte aligned, owned by the caller.  The library allocates
 *   nothing, copies nothing between host and device, never synchronises and
 *   keeps no global mutable state (kda_prefill_varlen_noalloc aside: it
 *   looks up, once per device, the address of the library's scratch array);
 *   it only enqueues kernels on `stream`
 *   (0 = the null stream), after reading the current device's compute-unit
 *   count and how many prefill workgroups a compute unit holds, which pick
 *   the launch shape of the bf16 prefill (the final states are the same bit
 *   for bit either way; the outputs may differ in their last bf16 place
 *   between shapes, since slices of one value tile group the chunk read-out
 *   differently from wider ones).  Buffers must stay valid until that work
 *   is done.
 * - log_alpha is the natural logarithm of the decay gate alpha (fp32, <= 0):
 *   alpha_t[i] in (0, 1) decays key channel i (the per-channel gate of the
 *   "Kimi Linear Guide" page, section "2. Channel-Wise Data-Dependent
 *   Gating").  The decode step takes any finite log_alpha.  The prefill
 *   forms each 64-token chunk's decay factors relative to its token 31, so
 *   it needs the gate sums over the 32 tokens on either side of that token
 *   to stay above -87 per channel (fp32 exponent range), which log_alpha in
 *   [-2.5, 0] guarantees.  A chunk outside that range is not rejected: its
 *   results may be non-finite and the call's status word reports it (see
 *   kda_prefill_status_offset).
 * - beta is one scalar write strength per token and head (§03).
 * - q, k, v, beta and o share one element type `dtype`; the state is fp32.
 * - State layout (init_state, final_state, decode state):
 *       state[n][h][j][i] = S_{ij}      i = key channel, j = value channel
 *   i.e. S^T row-major with the key index contiguous.  A prefill's final
 *   state can be fed unchanged to the decode step or to a later prefill.
 * - No query scaling is applied and q, k are used as given (the caller
 *   normalises keys, as §02 assumes).
 * - Validation happens on the host, before any HIP call, and returns a
 *   status; no exception or abort crosses this interface.  The contents of
 *   device arrays (cu_seqlens, gate values) are not inspected.
 * - Supported: dk == dv in {64, 128}; dtype KDA_BF16 or KDA_F32.
 * - Results are bitwise reproducible run to run on the same device: every
 *   sum has a fixed order; atomics only hand out work and publish
 *   readiness, never accumulate values.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL */
  KDA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  KDA_ERR_UNSUPPORTED = 3, /* head size not in {64, 128} or dk != dv */
  KDA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  KDA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  KDA_ERR_DTYPE = 6,       /* unknown element type */
  KDA_ERR_HIP = 7,         /* a kernel launch failed */
  KDA_ERR_SCRATCH = 8      /* sizes exceed kda_prefill_varlen_noalloc's scratch array */
} kda_status;

typedef enum kda_dtype {
  KDA_BF16 = 0, /* bfloat16 q, k, v, beta and o; fp32 state and accumulation */
  KDA_F32 = 1   /* float32 everywhere */
} kda_dtype;

/* Static description of a status code (never NULL). */
const char* kda_status_string(kda_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int kda_version(void);

/*
 * Bytes of device workspace kda_prefill_varlen needs for these sizes
 * (0 on invalid sizes).  Depends only on the arguments.  The workspace holds
 * per-chunk factors of the chunked form, and for bf16 one readiness flag
 * per (chunk, head) and a small header; its contents need not be
 * initialised on entry.  A workspace must not be shared by calls that may
 * run at the same time.
 */
size_t kda_prefill_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                  int32_t num_heads, int32_t dk, int32_t dv,
                                  kda_dtype dtype);

/*
 * Byte offset, inside the workspace of a prefill call with these sizes, of
 * an int32 status word that the call sets (SIZE_MAX on invalid sizes).  It
 * is meaningful once the call's work on the stream is done, for calls with
 * total_tokens > 0; the caller reads it when it wants to (it is not
 * returned, since the call does not wait for its kernels):
 *   0   the call went as intended;
 *   1   (bit 0) a wait of the bf16 path's state pass for a chunk's factors
 *       gave up after about two seconds -- the device was shared so heavily
 *       that the factors did not arrive; the affected sequences' outputs
 *       and final states are NaN;
 *   2   (bit 1) a chunk's decay factors left the fp32 range (gate sums
 *       below -87 on one side of the chunk's anchor token); its results
 *       may be non-finite.
 * The pooled, Gated DeltaNet and raw-input prefill forms use the same word.
 */
size_t kda_prefill_status_offset(int32_t num_seqs, int64_t total_tokens,
                                 int32_t num_heads, int32_t dk, int32_t dv,
                                 kda_dtype dtype);

/*
 * Chunk-parallel prefill over variable-length packed sequences
 * ("Kimi Delta Attention" §06, chunk-parallel mode; chunks of 64 tokens as
 * in the "Kimi Linear Guide" hardware-chunking section).  Sequence n
 * occupies tokens [cu_seqlens[n], cu_seqlens[n+1]); chunks start at each
 * sequence's first token and the last one may be partial.  Tokens of
 * different sequences never interact.
 *
 *   q, k        [total_tokens, num_heads, dk]  dtype
 *   v           [total_tokens, num_heads, dv]  dtype
 *   log_alpha   [total_tokens, num_heads, dk]  fp32
 *   beta        [total_tokens, num_heads]      dtype
 *   cu_seqlens  [num_seqs + 1] int32 device array: cu[0] = 0,
 *               non-decreasing, cu[num_seqs] = total_tokens (not checked)
 *   init_state  [num_seqs, num_heads, dv, dk] fp32, or NULL for zero states
 *   o           [total_tokens, num_heads, dv]  dtype (output)
 *   final_state [num_seqs, num_heads, dv, dk] fp32 (output), or NULL to skip.
 *               May equal init_state (in-place continuation); no other
 *               aliasing between arguments is allowed.
 *   workspace   device buffer of at least kda_prefill_workspace_size(...)
 *               bytes (16-byte aligned)
 *
 * A sequence of length 0 produces no outputs and final_state = init_state
 * (or zeros).  total_tokens may be 0.
 *
 * Precision of the bf16 path: fp32 accumulation; the sequential pass over
 * chunks multiplies fp16 operands (the per-chunk factors, the state and the
 * prediction error), so state entries and values must stay below 6.5e4 in
 * magnitude -- true for normalised keys and values of order one.  The fp32
 * path computes with fp32 operands throughout.
 */
kda_status kda_prefill_varlen(const void* q, const void* k, const void* v,
                              const float* log_alpha, const void* beta,
                              const int32_t* cu_seqlens,
                              const float* init_state,
                              void* o, float* final_state,
                              int32_t num_seqs, int64_t total_tokens,
                              int32_t num_heads, int32_t dk, int32_t dv,
                              kda_dtype dtype,
                              void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * One recurrent decode step for num_seqs sequences x num_heads heads
 * ("Kimi Delta Attention" §06, fused recurrent mode: decay, correct and
 * write the state in place, then read the output).
 *
 *   q, k       [num_seqs, num_heads, dk]  dtype
 *   v          [num_seqs, num_heads, dv]  dtype
 *   log_alpha  [num_seqs, num_heads, dk]  fp32
 *   beta       [num_seqs, num_heads]      dtype
 *   state      [num_seqs, num_heads, dv, dk] fp32, read and overwritten
 *   o          [num_seqs, num_heads, dv]  dtype (output)
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* log_alpha, const void* beta,
                           float* state, void* o,
                           int32_t num_seqs, int32_t num_heads,
                           int32_t dk, int32_t dv, kda_dtype dtype,
                           hipStream_t stream);

/*
 * Gated DeltaNet forms of the two calls: one decay gate per (token, head)
 * instead of one per key channel -- the scalar-gated delta rule that the
 * "Kimi Delta Attention" page (§02-§03) refines into KDA by giving every key
 * dimension its own gate.  With a scalar gate, alpha (I - beta k k^T) S =
 * (I - beta k k^T) alpha S, so the recurrence is KDA's with alpha_t[i] equal
 * for all i.  Arguments, layouts and errors as for the KDA calls, except:
 *
 *   log_alpha  [total_tokens, num_heads] fp32   (kda_gdn_prefill_varlen)
 *   log_alpha  [num_seqs, num_heads]     fp32   (kda_gdn_decode_step)
 *
 * The workspace is kda_prefill_workspace_size(...) as for KDA.
 */
kda_status kda_gdn_prefill_varlen(const void* q, const void* k, const void* v,
                                  const float* log_alpha, const void* beta,
                                  const int32_t* cu_seqlens,
                                  const float* init_state,
                                  void* o, float* final_state,
                                  int32_t num_seqs, int64_t total_tokens,
                                  int32_t num_heads, int32_t dk, int32_t dv,
                                  kda_dtype dtype,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

kda_status kda_gdn_decode_step(const void* q, const void* k, const void* v,
                               const float* log_alpha, const void* beta,
                               float* state, void* o,
                               int32_t num_seqs, int32_t num_heads,
                               int32_t dk, int32_t dv, kda_dtype dtype,
                               hipStream_t stream);

/*
 * Raw-input forms of the KDA calls: the kernels apply the layer's input
 * prologue themselves -- q and k are made unit length per (token, head),
 * x / max(|x|_2, 1e-12) in fp32, and beta is given as a logit and taken
 * through the sigmoid (the "Kimi Linear Guide" page, "End-to-End
 * Implementation": keys and queries normalised, the write strength squashed
 * to (0, 1); the "Kimi Delta Attention" page §02 assumes normalised keys).
 * Arguments, layouts and errors as for kda_prefill_varlen and
 * kda_decode_step, with beta_logit in place of beta.
 */
kda_status kda_prefill_varlen_raw(const void* q, const void* k, const void* v,
                                  const float* log_alpha, const void* beta_logit,
                                  const int32_t* cu_seqlens,
                                  const float* init_state,
                                  void* o, float* final_state,
                                  int32_t num_seqs, int64_t total_tokens,
                                  int32_t num_heads, int32_t dk, int32_t dv,
                                  kda_dtype dtype,
                                  void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

kda_status kda_decode_step_raw(const void* q, const void* k, const void* v,
                               const float* log_alpha, const void* beta_logit,
                               float* state, void* o,
                               int32_t num_seqs, int32_t num_heads,
                               int32_t dk, int32_t dv, kda_dtype dtype,
                               hipStream_t stream);

/*
 * State-pool forms of the two calls, for a serving engine that keeps every
 * live sequence's recurrent state in one caller-owned pool and checkpoints
 * prefixes ("Kimi Delta Attention" §07: the fixed-size state is the whole
 * per-sequence cache; a prefix is resumed from its saved state).
 *
 *   state_indices  [num_seqs] int32 device array: sequence n uses pool slot
 *                  state_indices[n].  Slots must be distinct within a call.
 *                  An index outside [0, pool_slots) is skipped on the
 *                  device: that sequence's state is neither read nor
 *                  written (prefill still writes its outputs, computed from
 *                  a zero initial state; decode leaves its outputs as they
 *                  were).
 *   state_pool     [pool_slots, num_heads, dv, dk] fp32, same per-slot
 *                  layout as the state arguments above.
 *
 * kda_prefill_varlen_pooled: as kda_prefill_varlen, with the initial state
 * of sequence n read from its slot when read_initial != 0 (zeros when 0)
 * and its final state written back to the slot.
 * kda_decode_step_pooled: as kda_decode_step, with the state of sequence n
 * read and overwritten in its slot.
 * Errors as for the plain calls; pool_slots < 0 is KDA_ERR_SHAPE and a NULL
 * state_indices or state_pool is KDA_ERR_NULL.
 */
kda_status kda_prefill_varlen_pooled(const void* q, const void* k, const void* v,
                                     const float* log_alpha, const void* beta,
                                     const int32_t* cu_seqlens,
                                     const int32_t* state_indices,
                                     float* state_pool, int32_t pool_slots,
                                     int32_t read_initial, void* o,
                                     int32_t num_seqs, int64_t total_tokens,
                                     int32_t num_heads, int32_t dk, int32_t dv,
                                     kda_dtype dtype,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

kda_status kda_decode_step_pooled(const void* q, const void* k, const void* v,
                                  const float* log_alpha, const void* beta,
                                  const int32_t* state_indices,
                                  float* state_pool, int32_t pool_slots, void* o,
                                  int32_t num_seqs, int32_t num_heads,
                                  int32_t dk, int32_t dv, kda_dtype dtype,
                                  hipStream_t stream);

/*
 * Backward pass of kda_prefill_varlen (training; "Kimi Delta Attention" §06
 * names training as the other user of the chunk-parallel form).  For a loss
 * L with upstream gradients grad_o = dL/do and grad_final_state = dL/dS_T it
 * writes the gradients of L with respect to every input of the forward call
 * on the same arguments.  The pages give no gradient; it is the reverse-mode
 * derivative of the recurrence above, organised by chunks of 64 tokens: a
 * forward pass re-derives every chunk's entering state, a reverse pass over
 * the chunks carries dL/dS, and each chunk then assembles its tokens'
 * gradients from its own factors.
 *
 *   q, k, v, log_alpha, beta, cu_seqlens, init_state, num_seqs, total_tokens,
 *   num_heads, dk, dv, dtype : exactly as passed to kda_prefill_varlen
 *                    (init_state may be NULL = zeros)
 *   grad_o           [T, H, dv] in `dtype` (required when T > 0)
 *   grad_final_state [N, H, dv, dk] fp32, or NULL (zero)
 *   grad_q, grad_k   [T, H, dk] fp32        (required when T > 0)
 *   grad_v           [T, H, dv] fp32        (required when T > 0)
 *   grad_log_alpha   [T, H, dk] fp32        (required when T > 0)
 *   grad_beta        [T, H]     fp32        (required when T > 0)
 *   grad_init_state  [N, H, dv, dk] fp32, or NULL (not written); it may be
 *                    the same buffer as grad_final_state, no other aliasing
 *   workspace        >= kda_prefill_backward_workspace_size(...) bytes of
 *                    device memory, contents irrelevant on entry.  It holds
 *                    the state entering every 64-token chunk (64 KiB per
 *                    (chunk, head) at dk = 128), one dL/dS per (sequence,
 *                    head), and the full factors of a window of at most 512
 *                    chunk slots and 8 GiB (0.93 MB per (chunk, head)); longer
 *                    calls run window by window, recomputing each window's
 *                    factors once more (17.5 GB for 16 sequences of 270,810
 *                    tokens at 32 heads, 24.8 GB for 2^20 tokens at 16).
 * Gradients are fp32 whatever `dtype` is.  Zero-length sequences give
 * grad_init_state = grad_final_state.  Errors as for kda_prefill_varlen.
 */
size_t kda_prefill_backward_workspace_size(int32_t num_seqs, int64_t total_tokens,
                                           int32_t num_heads, int32_t dk, int32_t dv,
                                           kda_dtype dtype);

kda_status kda_prefill_backward(const void* q, const void* k, const void* v,
                                const float* log_alpha, const void* beta,
                                const int32_t* cu_seqlens, const float* init_state,
                                const void* grad_o, const float* grad_final_state,
                                float* grad_q, float* grad_k, float* grad_v,
                                float* grad_log_alpha, float* grad_beta,
                                float* grad_init_state,
                                int32_t num_seqs, int64_t total_tokens,
                                int32_t num_heads, int32_t dk, int32_t dv,
                                kda_dtype dtype,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * kda_prefill_varlen without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The call itself allocates nothing (no
 * hipMalloc, no allocating library routine); its workspace is a device array
 * of KDA_NOALLOC_SCRATCH_BYTES bytes built into the library, of which each
 * GPU that runs the library holds one copy from the first load of the
 * library's kernels until the process ends.  Arguments, layouts and results
 * are exactly those of kda_prefill_varlen (same kernels).
 *
 * Limits and sharing: sizes whose kda_prefill_workspace_size(...) exceeds
 * KDA_NOALLOC_SCRATCH_BYTES return KDA_ERR_SCRATCH before any HIP call (for
 * bf16 and dk = 128 that is about 4,880 (64-token chunk, head) pairs, e.g.
 * 8K tokens of 32 heads in one sequence).  Every call on a GPU uses that
 * GPU's one array, so calls that may run at the same time on one GPU (on
 * different streams, or from different threads) race and must not be
 * issued; calls in one stream are ordered and safe.  Each call clears what
 * must start at zero itself.  The status word of kda_prefill_status_offset
 * lives in the array and is not exposed for these calls.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)384 << 20)

kda_status kda_prefill_varlen_noalloc(const void* q, const void* k, const void* v,
                                      const float* log_alpha, const void* beta,
                                      const int32_t* cu_seqlens,
                                      const float* init_state,
                                      void* o, float* final_state,
                                      int32_t num_seqs, int64_t total_tokens,
                                      int32_t num_heads, int32_t dk, int32_t dv,
                                      kda_dtype dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
