// kda_api.cpp -- the C ABI of include/kda.h: host-side validation (no HIP
// call happens before every check has passed), workspace sizing, and the
// hand-off to the kernel launchers.
#include "kda.h"

#include <stdint.h>

#include "kda_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kda_status check_common(int32_t num_seqs, int32_t num_heads, int32_t dk, int32_t dv,
                        kda_dtype dtype) {
  if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_DTYPE;
  if (num_seqs < 0 || num_heads <= 0 || dk <= 0 || dv <= 0) return KDA_ERR_SHAPE;
  if (dk != dv || (dk != 64 && dk != 128)) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

}  // namespace

namespace kda {

// Checks of a prefill call's arguments other than the workspace.
kda_status prefill_check(const void* q, const void* k, const void* v, const float* log_alpha, const void* beta,
                         const int32_t* cu_seqlens, const float* init_state, void* o, float* final_state,
                         int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                         kda_dtype dtype) {
  kda_status st = check_common(num_seqs, num_heads, dk, dv, dtype);
  if (st != KDA_OK) return st;
  if (num_seqs < 1 || total_tokens < 0 || total_tokens > INT32_MAX) return KDA_ERR_SHAPE;
  if (!cu_seqlens) return KDA_ERR_NULL;
  if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, log_alpha, beta, cu_seqlens, init_state, o, final_state};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  return KDA_OK;
}

kda_status prefill_call(const void* q, const void* k, const void* v,
                              const float* log_alpha, const void* beta,
                              const int32_t* cu_seqlens, const float* init_state,
                              void* o, float* final_state, int32_t num_seqs,
                              int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                              kda_dtype dtype, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, bool scalar_gate, bool raw) {
  kda_status st = kda::prefill_check(q, k, v, log_alpha, beta, cu_seqlens, init_state, o, final_state, num_seqs,
                                     total_tokens, num_heads, dk, dv, dtype);
  if (st != KDA_OK) return st;
  if (workspace && !aligned16(workspace)) return KDA_ERR_ALIGN;
  const size_t need = kda_prefill_workspace_size(num_seqs, total_tokens, num_heads, dk, dv, dtype);
  if (total_tokens > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;

  kda::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
  a.cu_seqlens = cu_seqlens; a.init_state = init_state; a.o = o; a.final_state = final_state;
  a.num_seqs = num_seqs; a.total_tokens = total_tokens; a.num_heads = num_heads; a.d = dk;
  a.bf16 = dtype == KDA_BF16; a.workspace = workspace;
  a.state_indices = nullptr; a.pool_slots = 0; a.scalar_gate = scalar_gate; a.raw_qkb = raw;
  const hipError_t e = a.bf16 ? kda::launch_prefill_bf16(a, stream) : kda::launch_prefill_f32(a, stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace kda

namespace {
using kda::prefill_call;

kda_status decode_plain(const void* q, const void* k, const void* v, const float* log_alpha,
                           const void* beta, float* state, void* o, int32_t num_seqs,
                           int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                           hipStream_t stream, bool scalar_gate, bool raw) {
  kda_status st = check_common(num_seqs, num_heads, dk, dv, dtype);
  if (st != KDA_OK) return st;
  if ((int64_t)num_seqs * num_heads > INT32_MAX) return KDA_ERR_SHAPE;
  if (num_seqs == 0) return KDA_OK;
  if (!q || !k || !v || !log_alpha || !beta || !state || !o) return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, log_alpha, beta, state, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return KDA_ERR_ALIGN;

  kda::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.state = state; a.o = o;
  a.num_seqs = num_seqs; a.num_heads = num_heads; a.d = dk; a.bf16 = dtype == KDA_BF16;
  a.state_indices = nullptr; a.pool_slots = 0; a.scalar_gate = scalar_gate; a.raw_qkb = raw;
  return kda::launch_decode(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case KDA_ERR_UNSUPPORTED: return "unsupported head size (dk == dv in {64, 128} required)";
    case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_DTYPE: return "unknown element type";
    case KDA_ERR_HIP: return "kernel launch failed";
    case KDA_ERR_SCRATCH: return "sizes exceed the no-allocation prefill's scratch array";
  }
  return "unknown status";
}

int kda_version(void) { return 100; }  // 0.1.0

size_t kda_prefill_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                  int32_t dk, int32_t dv, kda_dtype dtype) {
  if (check_common(num_seqs, num_heads, dk, dv, dtype) != KDA_OK) return 0;
  if (total_tokens < 0 || total_tokens > INT32_MAX) return 0;
  const int64_t slots = kda::prefill_num_slots(num_seqs, total_tokens);
  if (dtype == KDA_BF16) return kda::prefill_workspace_bytes_bf16(slots, num_heads, dk);
  return kda::prefill_status_offset_f32(slots, num_heads, dk) + 16;
}

size_t kda_prefill_status_offset(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t dk,
                                 int32_t dv, kda_dtype dtype) {
  if (kda_prefill_workspace_size(num_seqs, total_tokens, num_heads, dk, dv, dtype) == 0) return SIZE_MAX;
  const int64_t slots = kda::prefill_num_slots(num_seqs, total_tokens);
  return dtype == KDA_BF16 ? kda::prefill_status_offset_bf16(slots, num_heads, dk)
                           : kda::prefill_status_offset_f32(slots, num_heads, dk);
}

kda_status kda_prefill_varlen(const void* q, const void* k, const void* v,
                              const float* log_alpha, const void* beta,
                              const int32_t* cu_seqlens, const float* init_state,
                              void* o, float* final_state, int32_t num_seqs,
                              int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                              kda_dtype dtype, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  return prefill_call(q, k, v, log_alpha, beta, cu_seqlens, init_state, o, final_state, num_seqs,
                       total_tokens, num_heads, dk, dv, dtype, workspace, workspace_bytes, stream, false,
                       false);
}

kda_status kda_gdn_prefill_varlen(const void* q, const void* k, const void* v,
                                  const float* log_alpha, const void* beta,
                                  const int32_t* cu_seqlens, const float* init_state,
                                  void* o, float* final_state, int32_t num_seqs,
                                  int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                                  kda_dtype dtype, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  return prefill_call(q, k, v, log_alpha, beta, cu_seqlens, init_state, o, final_state, num_seqs,
                       total_tokens, num_heads, dk, dv, dtype, workspace, workspace_bytes, stream, true,
                       false);
}

kda_status kda_prefill_varlen_raw(const void* q, const void* k, const void* v,
                                  const float* log_alpha, const void* beta_logit,
                                  const int32_t* cu_seqlens, const float* init_state,
                                  void* o, float* final_state, int32_t num_seqs,
                                  int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                                  kda_dtype dtype, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  return prefill_call(q, k, v, log_alpha, beta_logit, cu_seqlens, init_state, o, final_state, num_seqs,
                       total_tokens, num_heads, dk, dv, dtype, workspace, workspace_bytes, stream, false,
                       true);
}

kda_status kda_prefill_varlen_pooled(const void* q, const void* k, const void* v,
                                     const float* log_alpha, const void* beta,
                                     const int32_t* cu_seqlens, const int32_t* state_indices,
                                     float* state_pool, int32_t pool_slots, int32_t read_initial,
                                     void* o, int32_t num_seqs, int64_t total_tokens,
                                     int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  kda_status st = check_common(num_seqs, num_heads, dk, dv, dtype);
  if (st != KDA_OK) return st;
  if (num_seqs < 1 || total_tokens < 0 || total_tokens > INT32_MAX || pool_slots < 0) return KDA_ERR_SHAPE;
  if (!cu_seqlens || !state_indices || !state_pool) return KDA_ERR_NULL;
  if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, log_alpha, beta, cu_seqlens, state_indices, state_pool, o, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  const size_t need = kda_prefill_workspace_size(num_seqs, total_tokens, num_heads, dk, dv, dtype);
  if (total_tokens > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;

  kda::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
  a.cu_seqlens = cu_seqlens; a.init_state = read_initial ? state_pool : nullptr; a.o = o;
  a.final_state = state_pool;
  a.num_seqs = num_seqs; a.total_tokens = total_tokens; a.num_heads = num_heads; a.d = dk;
  a.bf16 = dtype == KDA_BF16; a.workspace = workspace;
  a.state_indices = state_indices; a.pool_slots = pool_slots; a.scalar_gate = false; a.raw_qkb = false;
  const hipError_t e = a.bf16 ? kda::launch_prefill_bf16(a, stream) : kda::launch_prefill_f32(a, stream);
  return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                           const void* beta, float* state, void* o, int32_t num_seqs,
                           int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                           hipStream_t stream) {
  return decode_plain(q, k, v, log_alpha, beta, state, o, num_seqs, num_heads, dk, dv, dtype, stream, false,
                      false);
}

kda_status kda_decode_step_raw(const void* q, const void* k, const void* v, const float* log_alpha,
                               const void* beta_logit, float* state, void* o, int32_t num_seqs,
                               int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                               hipStream_t stream) {
  return decode_plain(q, k, v, log_alpha, beta_logit, state, o, num_seqs, num_heads, dk, dv, dtype, stream,
                      false, true);
}

kda_status kda_gdn_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                               const void* beta, float* state, void* o, int32_t num_seqs,
                               int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype,
                               hipStream_t stream) {
  return decode_plain(q, k, v, log_alpha, beta, state, o, num_seqs, num_heads, dk, dv, dtype, stream, true,
                      false);
}

kda_status kda_decode_step_pooled(const void* q, const void* k, const void* v, const float* log_alpha,
                                  const void* beta, const int32_t* state_indices, float* state_pool,
                                  int32_t pool_slots, void* o, int32_t num_seqs, int32_t num_heads,
                                  int32_t dk, int32_t dv, kda_dtype dtype, hipStream_t stream) {
  kda_status st = check_common(num_seqs, num_heads, dk, dv, dtype);
  if (st != KDA_OK) return st;
  if ((int64_t)num_seqs * num_heads > INT32_MAX || pool_slots < 0) return KDA_ERR_SHAPE;
  if (num_seqs == 0) return KDA_OK;
  if (!q || !k || !v || !log_alpha || !beta || !state_indices || !state_pool || !o) return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, log_alpha, beta, state_indices, state_pool, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return KDA_ERR_ALIGN;

  kda::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.state = state_pool; a.o = o;
  a.num_seqs = num_seqs; a.num_heads = num_heads; a.d = dk; a.bf16 = dtype == KDA_BF16;
  a.state_indices = state_indices; a.pool_slots = pool_slots; a.scalar_gate = false; a.raw_qkb = false;
  return kda::launch_decode(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_prefill_backward_workspace_size(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                           int32_t dk, int32_t dv, kda_dtype dtype) {
  if (check_common(num_seqs, num_heads, dk, dv, dtype) != KDA_OK) return 0;
  if (total_tokens < 0 || total_tokens > INT32_MAX) return 0;
  const int64_t slots = kda::prefill_num_slots(num_seqs, total_tokens);
  return kda::backward_workspace_bytes(num_seqs, slots, num_heads, dk);
}

kda_status kda_prefill_backward(const void* q, const void* k, const void* v, const float* log_alpha,
                                const void* beta, const int32_t* cu_seqlens, const float* init_state,
                                const void* grad_o, const float* grad_final_state, float* grad_q,
                                float* grad_k, float* grad_v, float* grad_log_alpha, float* grad_beta,
                                float* grad_init_state, int32_t num_seqs, int64_t total_tokens,
                                int32_t num_heads, int32_t dk, int32_t dv, kda_dtype dtype, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  kda_status st = check_common(num_seqs, num_heads, dk, dv, dtype);
  if (st != KDA_OK) return st;
  if (num_seqs < 1 || total_tokens < 0 || total_tokens > INT32_MAX) return KDA_ERR_SHAPE;
  if (!cu_seqlens) return KDA_ERR_NULL;
  if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !grad_o || !grad_q || !grad_k ||
                           !grad_v || !grad_log_alpha || !grad_beta))
    return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, log_alpha, beta, cu_seqlens, init_state, grad_o, grad_final_state, grad_q,
                        grad_k, grad_v, grad_log_alpha, grad_beta, grad_init_state, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  const size_t need = kda_prefill_backward_workspace_size(num_seqs, total_tokens, num_heads, dk, dv, dtype);
  if (total_tokens > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;

  kda::BackwardArgs a;
  a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.cu_seqlens = cu_seqlens;
  a.init_state = init_state; a.grad_o = grad_o; a.grad_final_state = grad_final_state;
  a.grad_q = grad_q; a.grad_k = grad_k; a.grad_v = grad_v; a.grad_log_alpha = grad_log_alpha;
  a.grad_beta = grad_beta; a.grad_init_state = grad_init_state;
  a.num_seqs = num_seqs; a.total_tokens = total_tokens; a.num_heads = num_heads; a.d = dk;
  a.bf16 = dtype == KDA_BF16; a.workspace = workspace;
  return kda::launch_backward(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"

