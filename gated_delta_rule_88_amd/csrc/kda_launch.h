// kda_launch.h -- host-side launch interface between the validated C ABI
// (kda_api.cpp) and the kernels.  Arguments arrive here already checked.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

struct DecodeArgs {
  const void *q, *k, *v;
  const float* log_alpha;
  const void* beta;
  float* state;
  void* o;
  int32_t num_seqs, num_heads, d;
  bool bf16;
  const int32_t* state_indices;   // NULL: sequence n uses state[n]
  int32_t pool_slots;
  bool scalar_gate;               // log_alpha holds one gate per (sequence, head)
  bool raw_qkb;                   // q, k unnormalised and beta a logit (normalised in the kernel)
};

struct PrefillArgs {
  const void *q, *k, *v;
  const float* log_alpha;
  const void* beta;
  const int32_t* cu_seqlens;
  const float* init_state;
  void* o;
  float* final_state;
  int32_t num_seqs;
  int64_t total_tokens;
  int32_t num_heads, d;
  bool bf16;
  void* workspace;
  const int32_t* state_indices;   // NULL: sequence n uses init_state[n] / final_state[n]
  int32_t pool_slots;
  bool scalar_gate;               // log_alpha holds one gate per (token, head)
  bool raw_qkb;                   // q, k unnormalised and beta a logit (normalised in the kernel)
};

struct BackwardArgs {
  const void *q, *k, *v;
  const float* log_alpha;
  const void* beta;
  const int32_t* cu_seqlens;
  const float* init_state;        // NULL: zero initial states
  const void* grad_o;             // dL/do, in the input type
  const float* grad_final_state;  // NULL: zero
  float *grad_q, *grad_k, *grad_v, *grad_log_alpha, *grad_beta;
  float* grad_init_state;         // NULL: not written
  int32_t num_seqs;
  int64_t total_tokens;
  int32_t num_heads, d;
  bool bf16;
  void* workspace;
};

// Per-chunk factor record of the prefill (bytes) for each precision path,
// and the number of chunk slots reserved for (num_seqs, total_tokens).
size_t prefill_record_bytes_f32(int d);
size_t prefill_record_bytes_bf16(int d);
// Whole workspace of the bf16 path: records, chunk-ready flags and a header;
// the byte offset of the call's status word in it.
size_t prefill_workspace_bytes_bf16(int64_t slots, int num_heads, int d);
size_t prefill_status_offset_bf16(int64_t slots, int num_heads, int d);
// fp32 path: records, then the status word (16-byte aligned, 16 bytes).
size_t prefill_status_offset_f32(int64_t slots, int num_heads, int d);
// Enqueues a kernel that sets *status to 0.
hipError_t clear_prefill_status(int* status, hipStream_t stream);
int64_t prefill_num_slots(int32_t num_seqs, int64_t total_tokens);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);

// The prefill behind every plain prefill entry point (kda_api.cpp): checks of
// the arguments other than the workspace, then the whole checked call.
kda_status prefill_check(const void* q, const void* k, const void* v, const float* log_alpha, const void* beta,
                         const int32_t* cu_seqlens, const float* init_state, void* o, float* final_state,
                         int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                         kda_dtype dtype);
kda_status prefill_call(const void* q, const void* k, const void* v, const float* log_alpha, const void* beta,
                        const int32_t* cu_seqlens, const float* init_state, void* o, float* final_state,
                        int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                        kda_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream,
                        bool scalar_gate, bool raw);

// Backward: workspace bytes for a call and the launcher.
size_t backward_workspace_bytes(int32_t num_seqs, int64_t slots, int num_heads, int d);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);

}  // namespace kda
