// kda_device.h -- device-side building blocks shared by the KDA kernels
// (gfx950 / CDNA4, wave64).
//
// MFMA fragment convention used everywhere in this library
// ---------------------------------------------------------
// All matrix products run on the 16x16 output MFMA family:
//   bf16:  v_mfma_f32_16x16x32_bf16  (one instruction per 32-deep block)
//   fp16:  v_mfma_f32_16x16x32_f16   (one instruction per 32-deep block)
//   fp32:  v_mfma_f32_16x16x4_f32    (eight instructions per 32-deep block)
// For a 32-deep reduction block, lane l (g = l / 16, r = l % 16) holds the
// row (A operand) or column (B operand) r of a 16-wide tile and eight
// reduction indices
//        kpos(g, m) = 4 g + (m & 3) + 16 (m >> 2),   m = 0..7.
// A and B use the same map, so any fixed assignment of reduction indices to
// (g, m) gives the same sum.  This particular one makes the accumulator of
// one product usable as the B operand of the next without moving data:
// the 16x16 accumulator layout gives lane l the rows 4 g + i (i = 0..3) of
// column r, so the two accumulator tiles covering rows [32p, 32p+16) and
// [32p+16, 32p+32) are, lane for lane, positions m = 0..3 and m = 4..7 of
// the fragment of reduction block p.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kChunk = 64;  // tokens per chunk
constexpr int kThreads = 256;

__device__ __forceinline__ int kpos(int g, int m) { return 4 * g + (m & 3) + 16 * (m >> 2); }

// ---------------------------------------------------------------------------
// Precision paths.  BF16: bf16 operands (split into hi + lo where the
// product feeds the recurrence), fp32 accumulation.  F32: fp32 operands.
// ---------------------------------------------------------------------------
struct PathBF16 {
  using In = __bf16;
  using Frag = bf16x8;
  using Half = bf16x4;
  static constexpr bool kSplit = true;
};
struct PathF32 {
  using In = float;
  using Frag = f32x8;
  using Half = f32x4;
  static constexpr bool kSplit = false;
};

__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

__device__ __forceinline__ void mma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const f16x8& a, const f16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int m = 0; m < 8; ++m) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[m], acc, 0, 0, 0);
}

// A fragment built from fp32 values, with its rounding residue when the
// path splits.  For the fp32 path lo stays unused.
template <class P>
struct Split {
  typename P::Frag hi, lo;
};

template <class P>
__device__ __forceinline__ Split<P> make_split(const float (&v)[8]) {
  Split<P> s;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    auto h = from_f32<typename P::In>(v[m]);
    s.hi[m] = h;
    if constexpr (P::kSplit) s.lo[m] = from_f32<typename P::In>(v[m] - to_f32(h));
  }
  return s;
}

template <class P>
__device__ __forceinline__ typename P::Frag make_frag(const float (&v)[8]) {
  typename P::Frag f;
#pragma unroll
  for (int m = 0; m < 8; ++m) f[m] = from_f32<typename P::In>(v[m]);
  return f;
}

// a*b with both operands split: hi*hi + hi*lo + lo*hi (lo*lo is below the
// fp32 rounding of the sum and skipped).
template <class P>
__device__ __forceinline__ void mma_ss(f32x4& acc, const Split<P>& a, const Split<P>& b) {
  mma(acc, a.hi, b.hi);
  if constexpr (P::kSplit) {
    mma(acc, a.hi, b.lo);
    mma(acc, a.lo, b.hi);
  }
}
// a split, b exact in the operand type.
template <class P>
__device__ __forceinline__ void mma_sx(f32x4& acc, const Split<P>& a, const typename P::Frag& b) {
  mma(acc, a.hi, b);
  if constexpr (P::kSplit) mma(acc, a.lo, b);
}
// a exact in the operand type, b split.
template <class P>
__device__ __forceinline__ void mma_xs(f32x4& acc, const typename P::Frag& a, const Split<P>& b) {
  mma(acc, a, b.hi);
  if constexpr (P::kSplit) mma(acc, a, b.lo);
}

// The input prologue of the raw-input calls: x / max(|x|, 1e-12) per
// (token, head) vector, and beta = 1 / (1 + e^-logit).
constexpr float kNormEps = 1e-12f;
__device__ __forceinline__ float inv_norm(float sumsq) { return 1.f / fmaxf(sqrtf(sumsq), kNormEps); }
__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row (lanes 16q .. 16q+15); every lane of
// the row receives the total.  xor-1 and xor-2 inside quads, then the
// half-row mirror and the row mirror pair the remaining groups.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

}  // namespace kda
