// kda_noalloc.hip -- kda_prefill_varlen_noalloc of include/kda.h: the
// prefill for callers that cannot allocate, with its workspace in a device
// array of the library.
#include <stdint.h>

#include <atomic>

#include <hip/hip_runtime.h>

#include "kda.h"
#include "kda_launch.h"

// ---------------------------------------------------------------------------
// Prefill without allocation.  Its workspace is a device array of this
// library: each GPU that runs the library holds its own copy (at its own
// address) until the process ends.  In host code the array's name is only a
// host-side stand-in, so the device address is looked up with
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever passed on (to the kernels, as the workspace).
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];   // per device; set once, never changed

kda_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return KDA_OK;
}
}  // namespace

kda_status kda_prefill_varlen_noalloc(const void* q, const void* k, const void* v,
                                      const float* log_alpha, const void* beta,
                                      const int32_t* cu_seqlens, const float* init_state,
                                      void* o, float* final_state, int32_t num_seqs,
                                      int64_t total_tokens, int32_t num_heads, int32_t dk, int32_t dv,
                                      kda_dtype dtype, hipStream_t stream) {
  kda_status st = kda::prefill_check(q, k, v, log_alpha, beta, cu_seqlens, init_state, o, final_state, num_seqs,
                                     total_tokens, num_heads, dk, dv, dtype);
  if (st != KDA_OK) return st;
  void* ws = nullptr;
  if (total_tokens > 0) {
    if (kda_prefill_workspace_size(num_seqs, total_tokens, num_heads, dk, dv, dtype) > KDA_NOALLOC_SCRATCH_BYTES)
      return KDA_ERR_SCRATCH;
    st = scratch_address(&ws);
    if (st != KDA_OK) return st;
  }
  return kda::prefill_call(q, k, v, log_alpha, beta, cu_seqlens, init_state, o, final_state, num_seqs, total_tokens,
                            num_heads, dk, dv, dtype, ws, KDA_NOALLOC_SCRATCH_BYTES, stream, false, false);
}
