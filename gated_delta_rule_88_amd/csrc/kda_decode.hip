// kda_decode.hip -- one recurrent KDA step per (sequence, head), in place.
//
// Operation (page "Kimi Delta Attention", §03 recurrence with the §02
// read-out; §06 "fused recurrent KDA": consume one q/k/v and gate set,
// decay, correct and write the state in place, read a fixed amount of
// recurrent memory).  With the state stored as S^T (row j = value channel j,
// key index i contiguous) and alpha = exp(log_alpha):
//
//   p_j   = sum_i S_ij alpha_i k_i          read of the decayed state at k
//   r_j   = sum_i S_ij alpha_i q_i          decayed state read at q
//   e_j   = beta (v_j - p_j)                scaled error
//   S_ij <- alpha_i S_ij + k_i e_j          decay + correction, in place
//   o_j   = r_j + (k . q) e_j               = (S_new^T q)_j
//
// Memory plan (HBM-bound: 2 x 64 KiB of state per head against 1.5 KiB of
// token data): one workgroup of 1024 threads per (sequence, head).  Sixteen
// lanes own one state row at a time, each lane D/16 keys as float4 pieces,
// so every load and store instruction of a wave moves four contiguous
// 256-byte row segments.  A thread issues all of its row loads before any
// arithmetic.  The state is streamed with nontemporal loads and stores (it
// is touched once per step and is larger than the caches).  The two dot
// products reduce over the 16 lanes of a DPP row; no LDS and no barrier.
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_prefill_common.h"

namespace kda {

constexpr int kDecodeThreads = 1024;

// SCALAR: one gate per (sequence, head); RAW: q, k unnormalised and beta a
// logit.  Compile-time, so the plain KDA step carries neither.
template <class P, int D, bool SCALAR, bool RAW>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(
    const typename P::In* __restrict__ q, const typename P::In* __restrict__ k,
    const typename P::In* __restrict__ v, const float* __restrict__ log_alpha,
    const typename P::In* __restrict__ beta, float* __restrict__ state,
    typename P::In* __restrict__ o, const int32_t* __restrict__ sidx, int pool_slots, int H) {
  using In = typename P::In;
  constexpr int NK = D / 16;        // keys per lane
  constexpr int NC = NK / 4;        // float4 pieces per lane and row
  constexpr int ROWS = D / (kDecodeThreads / 16);   // rows per 16-lane group

  const int64_t tok = blockIdx.x;   // n * H + h
  const int64_t slot = state_slot(sidx, pool_slots, (int)(tok / H));
  if (slot < 0) return;             // whole workgroup: no state for this sequence
  const int tid = threadIdx.x;
  const int grp = tid >> 4;         // groups of 16 lanes
  const int l16 = tid & 15;

  // token vectors for this lane's keys: c * 64 + 4 * l16 + {0..3}
  float a[NK], kk[NK], qq[NK], aq[NK], ak[NK];
  float ksq = 0.f, qsq = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int64_t base = tok * D + c * 64 + 4 * l16;
    f32x4 la;
    if constexpr (SCALAR) la = f32x4{log_alpha[tok], log_alpha[tok], log_alpha[tok], log_alpha[tok]};
    else la = *reinterpret_cast<const f32x4*>(log_alpha + base);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[4 * c + e] = __expf(la[e]);
      kk[4 * c + e] = to_f32(k[base + e]);
      qq[4 * c + e] = to_f32(q[base + e]);
      ksq += kk[4 * c + e] * kk[4 * c + e];
      qsq += qq[4 * c + e] * qq[4 * c + e];
    }
  }
  // raw inputs: unit q and k (each 16-lane row holds a whole token vector)
  float rk = 1.f, rq = 1.f;
  if constexpr (RAW) {
    rk = inv_norm(row16_sum(ksq));
    rq = inv_norm(row16_sum(qsq));
  }
  float kq_part = 0.f;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    kk[i] *= rk;
    const float qi = qq[i] * rq;
    ak[i] = a[i] * kk[i];
    aq[i] = a[i] * qi;
    kq_part += kk[i] * qi;
  }
  const float kq = row16_sum(kq_part);
  float b = to_f32(beta[tok]);
  if constexpr (RAW) b = sigmoid(b);

  float* srow0 = state + (slot * H + tok % H) * D * D;
  f32x4 s[ROWS][NC];
#pragma unroll
  for (int it = 0; it < ROWS; ++it) {
    const int j = grp * ROWS + it;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      s[it][c] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(srow0 + (int64_t)j * D + c * 64 + 4 * l16));
  }

  float my_o = 0.f;
#pragma unroll
  for (int it = 0; it < ROWS; ++it) {
    const int j = grp * ROWS + it;
    float pp = 0.f, rr = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pp += s[it][c][e] * ak[4 * c + e];
        rr += s[it][c][e] * aq[4 * c + e];
      }
    pp = row16_sum(pp);
    rr = row16_sum(rr);
    const float err = b * (to_f32(v[tok * D + j]) - pp);
    const float oj = rr + kq * err;
    if (l16 == it) my_o = oj;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      f32x4 ns;
#pragma unroll
      for (int e = 0; e < 4; ++e) ns[e] = a[4 * c + e] * s[it][c][e] + kk[4 * c + e] * err;
      __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(srow0 + (int64_t)j * D + c * 64 + 4 * l16));
    }
  }
  if (l16 < ROWS) o[tok * D + grp * ROWS + l16] = from_f32<In>(my_o);
}

template <class P, int D, bool SCALAR, bool RAW>
static hipError_t launch_decode_v(const DecodeArgs& A, hipStream_t stream) {
  using In = typename P::In;
  const unsigned blocks = (unsigned)((int64_t)A.num_seqs * A.num_heads);
  hipLaunchKernelGGL((decode_step_kernel<P, D, SCALAR, RAW>), dim3(blocks), dim3(kDecodeThreads), 0, stream,
                     (const In*)A.q, (const In*)A.k, (const In*)A.v, A.log_alpha,
                     (const In*)A.beta, A.state, (In*)A.o, A.state_indices, A.pool_slots, A.num_heads);
  return hipGetLastError();
}

template <class P, int D>
static hipError_t launch_decode_t(const DecodeArgs& A, hipStream_t stream) {
  if (A.scalar_gate) return launch_decode_v<P, D, true, false>(A, stream);
  if (A.raw_qkb) return launch_decode_v<P, D, false, true>(A, stream);
  return launch_decode_v<P, D, false, false>(A, stream);
}

hipError_t launch_decode(const DecodeArgs& A, hipStream_t stream) {
  if (A.num_seqs == 0) return hipSuccess;
  if (A.bf16) return A.d == 128 ? launch_decode_t<PathBF16, 128>(A, stream)
                                : launch_decode_t<PathBF16, 64>(A, stream);
  return A.d == 128 ? launch_decode_t<PathF32, 128>(A, stream)
                    : launch_decode_t<PathF32, 64>(A, stream);
}

}  // namespace kda
