// kda_prefill_common.h -- pieces shared by the prefill kernels: the chunk
// slot map of packed variable-length sequences and small LDS helpers.
#pragma once

#include "kda_device.h"

namespace kda {

// Chunk slots: chunk c of sequence n lives in slot cu[n]/64 + n + c.  Slots
// of different sequences never collide (floor(a/64) + ceil(L/64) <=
// floor((a+L)/64) + 1), and every slot is below T/64 + N + 1.

__device__ __forceinline__ int64_t slot_key(const int32_t* cu, int n) {
  return (int64_t)(cu[n] / kChunk) + n;
}

// slot -> (sequence, first token, length); false for an unused slot.
__device__ __forceinline__ bool decode_slot(const int32_t* __restrict__ cu, int N, int64_t slot,
                                            int& n, int64_t& t0, int& len) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (slot_key(cu, mid) <= slot) lo = mid; else hi = mid - 1;
  }
  n = lo;
  const int64_t c = slot - slot_key(cu, lo);
  const int64_t L = (int64_t)cu[lo + 1] - cu[lo];
  if (c < 0 || c * kChunk >= L) return false;
  t0 = cu[lo] + c * kChunk;
  len = (int)min<int64_t>(kChunk, L - c * kChunk);
  return true;
}

// State slot of sequence n: n itself, or state_indices[n] for a state pool
// of pool_slots entries; -1 when that index is out of range (the sequence's
// state is then neither read nor written).
__device__ __forceinline__ int64_t state_slot(const int32_t* __restrict__ sidx, int pool_slots, int n) {
  if (!sidx) return n;
  const int s = sidx[n];
  return (s >= 0 && s < pool_slots) ? s : -1;
}

// Status word of a prefill call (in its workspace; see the C ABI's
// kda_prefill_status_offset): zero when the call went as intended.
constexpr int kStatusWaitGaveUp = 1;   // a wait for a chunk's factors gave up (NaN results)
constexpr int kStatusGateRange = 2;    // a chunk's decay factors left the fp32 range
// The decay factors are anchored at token 31 of the chunk: e^(G - G[31]) and
// its inverse stay finite while |G - G[31]| <= 87 -- i.e. for log_alpha in
// [-2.5, 0] and, more generally, while the gate sums over the 32 tokens on
// either side of the anchor stay above -87.
constexpr float kMaxAnchoredExp = 87.f;

// four consecutive inputs of a token-major LDS row as fp32
__device__ __forceinline__ f32x4 lds4(const __bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }


template <class P>
__device__ __forceinline__ void store_split(unsigned char* hi_base, unsigned char* lo_base, size_t off,
                                            const Split<P>& s) {
  using Frag = typename P::Frag;
  *reinterpret_cast<Frag*>(hi_base + off) = s.hi;
  if constexpr (P::kSplit) *reinterpret_cast<Frag*>(lo_base + off) = s.lo;
}

}  // namespace kda
