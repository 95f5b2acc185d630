// Test doubles for the kernel launchers behind the C ABI, so that
// kda_api.cpp (argument checks, workspace sizing, hand-off) runs host-only
// under the address and undefined-behaviour sanitizers.  Each launcher only
// counts its calls; the sizing functions return fixed, plausible sizes.
#include "kda_launch.h"

namespace kda {

int g_launches = 0;

size_t prefill_record_bytes_f32(int d) { return d == 128 ? 200000 : 60000; }
size_t prefill_record_bytes_bf16(int d) { return d == 128 ? 82432 : 24832; }
int64_t prefill_num_slots(int32_t num_seqs, int64_t total_tokens) { return total_tokens / 64 + num_seqs + 1; }
size_t prefill_workspace_bytes_bf16(int64_t slots, int num_heads, int d) {
  return (size_t)slots * num_heads * (prefill_record_bytes_bf16(d) + 4) + 256;
}
size_t prefill_status_offset_bf16(int64_t slots, int num_heads, int d) {
  return prefill_workspace_bytes_bf16(slots, num_heads, d) - 252;
}
size_t prefill_status_offset_f32(int64_t slots, int num_heads, int d) {
  return (size_t)slots * num_heads * prefill_record_bytes_f32(d);
}
hipError_t clear_prefill_status(int*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill_f32(const PrefillArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill_bf16(const PrefillArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
size_t backward_workspace_bytes(int32_t num_seqs, int64_t slots, int num_heads, int d) {
  return ((size_t)slots * num_heads + num_seqs) * d * d * 4 + (size_t)4 * num_heads * 300000;
}
hipError_t launch_backward(const BackwardArgs&, hipStream_t) { ++g_launches; return hipSuccess; }

}  // namespace kda
