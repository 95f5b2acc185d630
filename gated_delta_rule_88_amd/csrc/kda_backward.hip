// kda_backward.hip -- gradients of the chunked varlen prefill (reverse mode).
//
// The forward map is the chunkwise form of the KDA recurrence (page "Kimi
// Delta Attention", §03 for the recurrence, §06 for chunk-parallel training
// and prefill).  For one chunk of C tokens entering with state S0
// (dk x dv), with G the inclusive cumulative log decay, a a per-channel
// anchor, gC the chunk's last row of G and gamma = exp(gC):
//
//   Ka = K e^(G-a), Kb = K e^(a-G), Qa = Q e^(G-a), Kg = K e^G, Qg = Q e^G,
//   Kc = K e^(gC-G);  A = strict_lower(Ka Kb^T), Bq = lower(Qa Kb^T),
//   T = (I + Diag(beta) A)^-1, Tb = T Diag(beta), W = Tb Kg, U = Tb V,
//   E = U - W S0,  O = Qg S0 + Bq E,  S_end = Diag(gamma) S0 + Kc^T E.
//
// Given dO and dS_end the chain rule gives, chunk by chunk (backwards):
//
//   dE  = Bq^T dO + Kc dS_end
//   dS0 = Diag(gamma) dS_end + Qg^T dO - W^T dE          (previous chunk's dS_end)
//
// and, per chunk and in parallel once S0, dS_end, E, dE are known:
//
//   dQg = dO S0^T, dKc = E dS_end^T, dW = -dE S0^T, dBq = lower(dO E^T),
//   P = T^T dE, R = T^T dW, dV = Diag(beta) P, dKg = Diag(beta) R,
//   dT = dE (Diag(beta) V)^T + dW (Diag(beta) Kg)^T, dM = -T^T dT T^T,
//   dA = strict_lower(Diag(beta) dM),
//   dbeta = rowsum(P o V) + rowsum(R o Kg) + rowsum(strict_lower(dM) o A),
//   dKa = dA Kb, dKb = dA^T Ka + dBs^T Qa, dQa = dBs Kb  (dBs: dBq without
//   its diagonal, whose q_r . k_r terms carry no decay),
//   dK = dKa e^(G-a) + dKb e^(a-G) + dKg e^G + dKc e^(gC-G) + diag(dBq) Q,
//   dQ = dQa e^(G-a) + dQg e^G + diag(dBq) K,
//   dG = dKa o Ka - dKb o Kb + dQa o Qa + dKg o Kg + dQg o Qg - dKc o Kc,
//   dgC = colsum(dKc o Kc) + rowsum(dS_end o S0) o gamma,
//   dlog_alpha[r] = sum_{s >= r} dG[s] + dgC.
//
// Kernels (all fp32, products on v_mfma_f32_16x16x4_f32):
//   1. bwd_prep   one workgroup per (chunk, head): padded fp32 copies of the
//                 inputs, the factors above, T by column-wise substitution;
//   2. bwd_fwd    one workgroup per (sequence, head, 16 value columns): the
//                 forward state pass, storing S0 and E of every chunk;
//   3. bwd_dstate same split, chunks in reverse: stores dS_end and dE of every
//                 chunk and the gradient of the initial state;
//   4. bwd_grad   one workgroup per (chunk, head): the per-chunk products and
//                 the element-wise assembly of dq, dk, dv, dbeta, dlog_alpha.
// The kernels run over windows of chunk slots.  Everything per chunk lives in
// a per-(chunk, head) block of the window, except the state entering each
// chunk (S0), which is kept for every chunk of the call (64 KiB per (chunk,
// head) at d = 128, against about 1 MB for a block).  A forward sweep over
// the windows (prep, forward pass) stores S0; a reverse sweep then, window by
// window from the last, recomputes the window's blocks (prep and forward pass
// again from the stored S0, the same bits; the last window's blocks are still
// in place), runs the reverse pass with dL/dS carried between windows, and
// assembles the window's gradients.  One window covers every slot when the
// blocks fit the window budget.
#include <algorithm>

#include "kda_launch.h"
#include "kda_prefill_common.h"

namespace kda {
namespace bwd {

constexpr int C = kChunk;

// Per-(chunk, head) workspace block, in floats.  Row-major [rows][cols];
// DS (and the stored S0 of every chunk, outside the blocks) are stored like
// the states: [value column][key].  EG, EC, EGA,
// EAG hold e^G, e^(gC-G), e^(G-a), e^(a-G) and GAM e^gC, each evaluated in
// fp64 and rounded once.  The key gradient is kept in two parts, DKP =
// dKa e^(G-a) + dKg e^G and DKM = dKb e^(a-G) + dKc e^(gC-G): every
// decay-scaled operand is an input times its factor, so the gradient of the
// cumulative decay is dG = K o (DKP - DKM) + Q o DQ, formed in fp64 where it
// is summed.
template <int D>
struct Ws {
  static constexpr int64_t CD = (int64_t)C * D, CC = (int64_t)C * C, DD = (int64_t)D * D;
  static constexpr int64_t KX = 0, QX = CD, VX = 2 * CD, DOX = 3 * CD, KA = 4 * CD, KB = 5 * CD, QA = 6 * CD,
                           KG = 7 * CD, QG = 8 * CD, KC = 9 * CD, EG = 10 * CD, EC = 11 * CD, EGA = 12 * CD,
                           EAG = 13 * CD, W = 14 * CD, U = 15 * CD, E = 16 * CD, DE = 17 * CD, DQ = 18 * CD,
                           DKP = 19 * CD, DKM = 20 * CD, DW = 21 * CD;
  static constexpr int64_t A = 22 * CD, BQ = A + CC, T = BQ + CC, TB = T + CC, DBQ = TB + CC, DT = DBQ + CC,
                           X = DT + CC, DA = X + CC, DMA = DA + CC;
  static constexpr int64_t DS = DMA + CC;
  static constexpr int64_t BETA = DS + DD, DBQD = BETA + C, GAM = DBQD + C;
  static constexpr int64_t FLOATS = GAM + D;
  static_assert(FLOATS % 4 == 0, "blocks stay 16-byte aligned");
};

// A window of chunk slots [slot_lo, slot_hi) and the workspace regions.
struct Win {
  int64_t slot_lo, slot_hi;
  float* blocks;   // block of (slot, head): blocks + ((slot - slot_lo) * H + head) * FLOATS
  float* s0;       // [slots][H][dv][dk]: the state entering every chunk of the call
  float* carry;    // [N][H][dv][dk]: dL/dS handed from a window to the one before it
};

// A strided fp32 matrix view: element (i, j) at p[i * rs + j * cs]; one of
// rs, cs is 1 and the other a multiple of 4.
struct Mat {
  const float* p;
  int rs, cs;
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// The product helpers below are not inlined, so their pointer arguments
// reach them without an address space, and the compiler would use flat
// accesses (counted on both the vector-memory and the LDS counters, so
// every wait covers both).  They state the space instead: workspace and
// outputs are global memory, the panels and accumulators LDS.
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) const float gcfloat;
typedef __attribute__((address_space(1))) const f32x4 gcf32x4;
typedef __attribute__((address_space(3))) float lfloat;
typedef __attribute__((address_space(3))) f32x4 lf32x4;
__device__ __forceinline__ gfloat* glb(float* p) { return (gfloat*)p; }
__device__ __forceinline__ gcfloat* glb(const float* p) { return (gcfloat*)p; }
__device__ __forceinline__ f32x4 ld4(const float* p) { return *(gcf32x4*)p; }
__device__ __forceinline__ lfloat* loc(float* p) { return (lfloat*)p; }

// out (64 x N) = A (64 x Kd) B (Kd x N) by the whole workgroup (wave w owns
// output rows [16 w, 16 w + 16)); Kd a multiple of 32.  Panels of 32
// reduction indices are staged in LDS, reduction-index major, so that every
// MFMA operand read is conflict-free.  epi(row, col, value) is called once
// per output element, by the lane that owns it.  Begins and ends with a
// barrier, so the epilogue's writes are visible to the next call.
constexpr int kGemmLds = 32 * 80 + 32 * 144;   // floats, for N <= 128

template <int N, class Epi>
__device__ __attribute__((noinline)) void wg_gemm(const Mat A, const Mat B, int Kd, float* lds, Epi epi) {
  constexpr int LA = 80, LB = N + 16, NBQ = 8 * N / 256;
  lfloat* sA = loc(lds);
  lfloat* sB = loc(lds) + 32 * LA;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
  f32x4 acc[N / 16];
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // 32-deep panels of A and B in registers, two sets in turn: each panel is
  // loaded two panels ahead, so the loads of the next two are in flight
  // while one is multiplied
  f32x4 ra0[2], rb0[NBQ], ra1[2], rb1[NBQ];
  auto load = [&](int k0, f32x4 (&ra)[2], f32x4 (&rb)[NBQ]) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = tid + 256 * it;
      ra[it] = A.cs == 1 ? ld4(A.p + (int64_t)(idx & 63) * A.rs + k0 + 4 * (idx >> 6))
                         : ld4(A.p + (int64_t)(k0 + (idx >> 4)) * A.cs + 4 * (idx & 15));
    }
#pragma unroll
    for (int it = 0; it < NBQ; ++it) {
      const int idx = tid + 256 * it;
      rb[it] = B.cs == 1 ? ld4(B.p + (int64_t)(k0 + idx / (N / 4)) * B.rs + 4 * (idx % (N / 4)))
                         : ld4(B.p + (int64_t)(idx % N) * B.cs + k0 + 4 * (idx / N));
    }
  };
  auto panel = [&](int k0, f32x4 (&ra)[2], f32x4 (&rb)[NBQ]) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = tid + 256 * it;
      if (A.cs == 1) {   // reduction index contiguous in memory
        const int r = idx & 63, kq = idx >> 6;
#pragma unroll
        for (int i = 0; i < 4; ++i) sA[(4 * kq + i) * LA + r] = ra[it][i];
      } else {           // row index contiguous
        *(lf32x4*)(sA + (idx >> 4) * LA + 4 * (idx & 15)) = ra[it];
      }
    }
#pragma unroll
    for (int it = 0; it < NBQ; ++it) {
      const int idx = tid + 256 * it;
      if (B.cs == 1) {   // column index contiguous
        *(lf32x4*)(sB + (idx / (N / 4)) * LB + 4 * (idx % (N / 4))) = rb[it];
      } else {           // reduction index contiguous
        const int n = idx % N, kq = idx / N;
#pragma unroll
        for (int i = 0; i < 4; ++i) sB[(4 * kq + i) * LB + n] = rb[it][i];
      }
    }
    __syncthreads();
    if (k0 + 64 < Kd) load(k0 + 64, ra, rb);
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      const float a = sA[(kk + g) * LA + 16 * w + l16];
#pragma unroll
      for (int nt = 0; nt < N / 16; ++nt) acc[nt] = mfma4(a, sB[(kk + g) * LB + 16 * nt + l16], acc[nt]);
    }
    __syncthreads();
  };
  __syncthreads();   // operands written just before by other threads are visible
  load(0, ra0, rb0);
  if (32 < Kd) load(32, ra1, rb1);
  for (int k0 = 0; k0 < Kd; k0 += 64) {
    panel(k0, ra0, rb0);
    if (k0 + 32 < Kd) panel(k0 + 32, ra1, rb1);
  }
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) epi(16 * w + 4 * g + i, 16 * nt + l16, acc[nt][i]);
  __syncthreads();
}

// The same product with the accumulators returned to the caller (inlined, so
// they stay in registers): acc (64 x N) = A1 B1 (+ A2 B2 when K2 > 0), lane
// layout as above (rows 16 w + 4 g + i, columns 16 nt + l16).  Begins and
// ends with a barrier.
template <int N>
__device__ __forceinline__ void wg_mm(const Mat A1, const Mat B1, int K1, const Mat A2, const Mat B2, int K2,
                                      float* lds, f32x4 (&acc)[N / 16]) {
  constexpr int LA = 80, LB = N + 16, NBQ = 8 * N / 256;
  lfloat* sA = loc(lds);
  lfloat* sB = loc(lds) + 32 * LA;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 ra[2], rb[NBQ];
  bool a_kc = true, b_nc = true;   // layouts of the panel in the registers
  auto load = [&](int k0) {
    const bool first = k0 < K1;
    const Mat A = first ? A1 : A2, B = first ? B1 : B2;
    const int kk = first ? k0 : k0 - K1;
    a_kc = A.cs == 1;
    b_nc = B.cs == 1;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = tid + 256 * it;
      ra[it] = a_kc ? ld4(A.p + (int64_t)(idx & 63) * A.rs + kk + 4 * (idx >> 6))
                    : ld4(A.p + (int64_t)(kk + (idx >> 4)) * A.cs + 4 * (idx & 15));
    }
#pragma unroll
    for (int it = 0; it < NBQ; ++it) {
      const int idx = tid + 256 * it;
      rb[it] = b_nc ? ld4(B.p + (int64_t)(kk + idx / (N / 4)) * B.rs + 4 * (idx % (N / 4)))
                    : ld4(B.p + (int64_t)(idx % N) * B.cs + kk + 4 * (idx / N));
    }
  };
  __syncthreads();
  load(0);
  const int Kd = K1 + K2;
  for (int k0 = 0; k0 < Kd; k0 += 32) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = tid + 256 * it;
      if (a_kc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sA[(4 * (idx >> 6) + i) * LA + (idx & 63)] = ra[it][i];
      } else {
        *(lf32x4*)(sA + (idx >> 4) * LA + 4 * (idx & 15)) = ra[it];
      }
    }
#pragma unroll
    for (int it = 0; it < NBQ; ++it) {
      const int idx = tid + 256 * it;
      if (b_nc) {
        *(lf32x4*)(sB + (idx / (N / 4)) * LB + 4 * (idx % (N / 4))) = rb[it];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) sB[(4 * (idx / N) + i) * LB + idx % N] = rb[it][i];
      }
    }
    __syncthreads();
    if (k0 + 32 < Kd) load(k0 + 32);
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      const float a = sA[(kk + g) * LA + 16 * w + l16];
#pragma unroll
      for (int nt = 0; nt < N / 16; ++nt) acc[nt] = mfma4(a, sB[(kk + g) * LB + 16 * nt + l16], acc[nt]);
    }
    __syncthreads();
  }
}

// Two products with a shared right operand, out1 = A1 B and out2 = A2 B
// (each 64 x N, K a multiple of 32), in the lane layout of wg_mm: B's panels
// are loaded and staged once for both.  Uses kGemmLds2 floats of LDS.
constexpr int kGemmLds2 = 2 * 32 * 80 + 32 * 144;

template <int N>
__device__ __forceinline__ void wg_mm2(const Mat A1, const Mat A2, const Mat B, int K, float* lds,
                                       f32x4 (&acc1)[N / 16], f32x4 (&acc2)[N / 16]) {
  constexpr int LA = 80, LB = N + 16, NBQ = 8 * N / 256;
  lfloat* sA1 = loc(lds);
  lfloat* sA2 = loc(lds) + 32 * LA;
  lfloat* sB = loc(lds) + 64 * LA;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt) acc1[nt] = acc2[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 ra1[2], ra2[2], rb[NBQ];
  auto loadA = [&](const Mat& A, f32x4 (&ra)[2], int k0) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = tid + 256 * it;
      ra[it] = A.cs == 1 ? ld4(A.p + (int64_t)(idx & 63) * A.rs + k0 + 4 * (idx >> 6))
                         : ld4(A.p + (int64_t)(k0 + (idx >> 4)) * A.cs + 4 * (idx & 15));
    }
  };
  auto load = [&](int k0) {
    loadA(A1, ra1, k0);
    loadA(A2, ra2, k0);
#pragma unroll
    for (int it = 0; it < NBQ; ++it) {
      const int idx = tid + 256 * it;
      rb[it] = B.cs == 1 ? ld4(B.p + (int64_t)(k0 + idx / (N / 4)) * B.rs + 4 * (idx % (N / 4)))
                         : ld4(B.p + (int64_t)(idx % N) * B.cs + k0 + 4 * (idx / N));
    }
  };
  auto stageA = [&](const Mat& A, const f32x4 (&ra)[2], lfloat* sA) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = tid + 256 * it;
      if (A.cs == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sA[(4 * (idx >> 6) + i) * LA + (idx & 63)] = ra[it][i];
      } else {
        *(lf32x4*)(sA + (idx >> 4) * LA + 4 * (idx & 15)) = ra[it];
      }
    }
  };
  __syncthreads();
  load(0);
  for (int k0 = 0; k0 < K; k0 += 32) {
    stageA(A1, ra1, sA1);
    stageA(A2, ra2, sA2);
#pragma unroll
    for (int it = 0; it < NBQ; ++it) {
      const int idx = tid + 256 * it;
      if (B.cs == 1) {
        *(lf32x4*)(sB + (idx / (N / 4)) * LB + 4 * (idx % (N / 4))) = rb[it];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) sB[(4 * (idx / N) + i) * LB + idx % N] = rb[it][i];
      }
    }
    __syncthreads();
    if (k0 + 32 < K) load(k0 + 32);
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      const float a1 = sA1[(kk + g) * LA + 16 * w + l16], a2 = sA2[(kk + g) * LA + 16 * w + l16];
#pragma unroll
      for (int nt = 0; nt < N / 16; ++nt) {
        const float b = sB[(kk + g) * LB + 16 * nt + l16];
        acc1[nt] = mfma4(a1, b, acc1[nt]);
        acc2[nt] = mfma4(a2, b, acc2[nt]);
      }
    }
    __syncthreads();
  }
}

// Two products with a shared left operand, out1 = A B1 and out2 = A B2, the
// counterpart of wg_mm2.  Uses kGemmLds3 floats of LDS.
constexpr int kGemmLds3 = 32 * 80 + 2 * 32 * 144;

template <int N>
__device__ __forceinline__ void wg_mm2b(const Mat A, const Mat B1, const Mat B2, int K, float* lds,
                                        f32x4 (&acc1)[N / 16], f32x4 (&acc2)[N / 16]) {
  constexpr int LA = 80, LB = N + 16, NBQ = 8 * N / 256;
  lfloat* sA = loc(lds);
  lfloat* sB1 = loc(lds) + 32 * LA;
  lfloat* sB2 = sB1 + 32 * LB;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt) acc1[nt] = acc2[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 ra[2], rb1[NBQ], rb2[NBQ];
  auto loadB = [&](const Mat& B, f32x4 (&rb)[NBQ], int k0) {
#pragma unroll
    for (int it = 0; it < NBQ; ++it) {
      const int idx = tid + 256 * it;
      rb[it] = B.cs == 1 ? ld4(B.p + (int64_t)(k0 + idx / (N / 4)) * B.rs + 4 * (idx % (N / 4)))
                         : ld4(B.p + (int64_t)(idx % N) * B.cs + k0 + 4 * (idx / N));
    }
  };
  auto load = [&](int k0) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = tid + 256 * it;
      ra[it] = A.cs == 1 ? ld4(A.p + (int64_t)(idx & 63) * A.rs + k0 + 4 * (idx >> 6))
                         : ld4(A.p + (int64_t)(k0 + (idx >> 4)) * A.cs + 4 * (idx & 15));
    }
    loadB(B1, rb1, k0);
    loadB(B2, rb2, k0);
  };
  auto stageB = [&](const Mat& B, const f32x4 (&rb)[NBQ], lfloat* sB) {
#pragma unroll
    for (int it = 0; it < NBQ; ++it) {
      const int idx = tid + 256 * it;
      if (B.cs == 1) {
        *(lf32x4*)(sB + (idx / (N / 4)) * LB + 4 * (idx % (N / 4))) = rb[it];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) sB[(4 * (idx / N) + i) * LB + idx % N] = rb[it][i];
      }
    }
  };
  __syncthreads();
  load(0);
  for (int k0 = 0; k0 < K; k0 += 32) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = tid + 256 * it;
      if (A.cs == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sA[(4 * (idx >> 6) + i) * LA + (idx & 63)] = ra[it][i];
      } else {
        *(lf32x4*)(sA + (idx >> 4) * LA + 4 * (idx & 15)) = ra[it];
      }
    }
    stageB(B1, rb1, sB1);
    stageB(B2, rb2, sB2);
    __syncthreads();
    if (k0 + 32 < K) load(k0 + 32);
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      const float a = sA[(kk + g) * LA + 16 * w + l16];
#pragma unroll
      for (int nt = 0; nt < N / 16; ++nt) {
        acc1[nt] = mfma4(a, sB1[(kk + g) * LB + 16 * nt + l16], acc1[nt]);
        acc2[nt] = mfma4(a, sB2[(kk + g) * LB + 16 * nt + l16], acc2[nt]);
      }
    }
    __syncthreads();
  }
}

constexpr Mat kNoMat = {nullptr, 1, 1};

// What the epilogue of a 64 x D product does with acc, the product (every
// part optional; store, out, x and fx are row-major [C][D] arrays of the
// workspace block, or outputs, in global memory):
//   store = acc * store_scale;  out[(row) * out_rs + col] = beta_row * acc
//   for rows < len (the value gradient, straight into the output);
//   x  = (x_add ? x : 0) + s_row * acc * fx
//   rowsum[row] = sum over columns of acc * rf        (fp32, LDS [C])
//   colsum[(4 w + g) * D + col] = sum over the lane's four rows of acc * cf
//                                 (fp64, LDS [16][D]: one partial per
//                                 (wave, lane group); their sum is the
//                                 column sum)
// with s_row = beta_row when row_beta, else 1.  Each part loads everything
// it needs (half a tile at a time) before its first store, so a lane keeps
// its loads in flight.
struct EpiD {
  float* store = nullptr;
  float store_scale = 1.f;
  float* out = nullptr;
  int64_t out_rs = 0;
  int len = 0;
  float* x = nullptr;
  const float* fx = nullptr;
  bool x_add = false;
  bool row_beta = false;
  const float* beta = nullptr;
  float* rowsum = nullptr;
  const float* rf = nullptr;
  double* colsum = nullptr;
  const float* cf = nullptr;
};

template <int D>
__device__ __forceinline__ void epilogue_d(const f32x4 (&acc)[D / 16], const EpiD& e) {
  constexpr int NT = D / 16;
  const int tid = threadIdx.x, w = tid >> 6, g = (tid & 63) >> 4, l16 = tid & 15;
  const int64_t lane = (int64_t)(16 * w + 4 * g) * D + l16;   // this lane's first element
  gcfloat* beta = glb(e.beta);
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = e.row_beta ? beta[16 * w + 4 * g + i] : 1.f;
  if (e.store) {
    gfloat* st = glb(e.store);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[lane + i * D + 16 * nt] = e.store_scale * acc[nt][i];
  }
  if (e.out) {
    gfloat* out = glb(e.out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g + i;
      const float b = beta[r];
      if (r < e.len)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) out[r * e.out_rs + 16 * nt + l16] = b * acc[nt][i];
    }
  }
  constexpr int NH = NT > 4 ? NT / 2 : NT;   // the read-modify-write goes half a tile at a time
  if (e.x) {
    gcfloat* fx = glb(e.fx);
    gfloat* x = glb(e.x);
#pragma unroll
    for (int n0 = 0; n0 < NT; n0 += NH) {
      f32x4 f[NH], xv[NH];
#pragma unroll
      for (int nt = 0; nt < NH; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[nt][i] = fx[lane + i * D + 16 * (n0 + nt)];
          xv[nt][i] = e.x_add ? x[lane + i * D + 16 * (n0 + nt)] : 0.f;
        }
#pragma unroll
      for (int nt = 0; nt < NH; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[lane + i * D + 16 * (n0 + nt)] = xv[nt][i] + s[i] * acc[n0 + nt][i] * f[nt][i];
    }
  }
  if (e.rowsum) {
    gcfloat* rf = glb(e.rf);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n0 = 0; n0 < NT; n0 += NH) {
      f32x4 f[NH];
#pragma unroll
      for (int nt = 0; nt < NH; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) f[nt][i] = rf[lane + i * D + 16 * (n0 + nt)];
#pragma unroll
      for (int nt = 0; nt < NH; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[i] += acc[n0 + nt][i] * f[nt][i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // across the 16 lanes that hold the row
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) part[i] += __shfl_xor(part[i], m);
      if (l16 == 0) loc(e.rowsum)[16 * w + 4 * g + i] = part[i];
    }
  }
  if (e.colsum) {
    gcfloat* cf = glb(e.cf);
    __attribute__((address_space(3))) double* cs = (__attribute__((address_space(3))) double*)e.colsum;
#pragma unroll
    for (int n0 = 0; n0 < NT; n0 += NH) {
      f32x4 f[NH];
#pragma unroll
      for (int nt = 0; nt < NH; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) f[nt][i] = cf[lane + i * D + 16 * (n0 + nt)];
#pragma unroll
      for (int nt = 0; nt < NH; ++nt) {
        double t = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) t += (double)acc[n0 + nt][i] * (double)f[nt][i];
        cs[(4 * w + g) * D + 16 * (n0 + nt) + l16] = t;
      }
    }
  }
}

template <int D>
__device__ __attribute__((noinline)) void gemm_d(const Mat A1, const Mat B1, int K1, const Mat A2, const Mat B2,
                                                 int K2, float* lds, const EpiD e) {
  f32x4 acc[D / 16];
  wg_mm<D>(A1, B1, K1, A2, B2, K2, lds, acc);
  epilogue_d<D>(acc, e);
}

// out1 = A1 B and out2 = A2 B, each with its own epilogue.
template <int D>
__device__ __attribute__((noinline)) void gemm_d2(const Mat A1, const Mat A2, const Mat B, int K, float* lds,
                                                  const EpiD e1, const EpiD e2) {
  f32x4 acc1[D / 16], acc2[D / 16];
  wg_mm2<D>(A1, A2, B, K, lds, acc1, acc2);
  epilogue_d<D>(acc1, e1);
  epilogue_d<D>(acc2, e2);
}

// out1 = A1 B and out2 = A2 B added to two sums with the same factor:
// x1 += p1 fx and x2 += p2 fx (no row scale), fx loaded once.
template <int D>
__device__ __attribute__((noinline)) void gemm_d2_addf(const Mat A1, const Mat A2, const Mat B, int K, float* lds,
                                                       float* x1, float* x2, const float* fx) {
  constexpr int NT = D / 16, NH = NT > 4 ? NT / 2 : NT;
  f32x4 acc1[NT], acc2[NT];
  wg_mm2<D>(A1, A2, B, K, lds, acc1, acc2);
  const int tid = threadIdx.x, w = tid >> 6, g = (tid & 63) >> 4, l16 = tid & 15;
  const int64_t lane = (int64_t)(16 * w + 4 * g) * D + l16;
  gcfloat* f = glb(fx);
  gfloat* y1 = glb(x1);
  gfloat* y2 = glb(x2);
#pragma unroll
  for (int n0 = 0; n0 < NT; n0 += NH) {
    f32x4 fv[NH], v1[NH], v2[NH];
#pragma unroll
    for (int nt = 0; nt < NH; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t o = lane + i * D + 16 * (n0 + nt);
        fv[nt][i] = f[o];
        v1[nt][i] = y1[o];
        v2[nt][i] = y2[o];
      }
#pragma unroll
    for (int nt = 0; nt < NH; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t o = lane + i * D + 16 * (n0 + nt);
        y1[o] = v1[nt][i] + acc1[n0 + nt][i] * fv[nt][i];
        y2[o] = v2[nt][i] + acc2[n0 + nt][i] * fv[nt][i];
      }
  }
}

// x = p1 fx1 + p2 fx2 for two products p1 = A1 B1 (K1) and p2 = A2 B2 +
// A3 B3 (K2 each) computed one after the other, x written once (no
// read-modify-write); e1 also carries p1's other epilogue parts (e1.x and
// e1.fx are x and fx1).
template <int D>
__device__ __attribute__((noinline)) void gemm_d_sum2(const Mat A1, const Mat B1, int K1, const Mat A2, const Mat B2,
                                                      const Mat A3, const Mat B3, int K2, const float* fx2,
                                                      float* lds, const EpiD e1) {
  constexpr int NT = D / 16, NH = NT > 4 ? NT / 2 : NT;
  f32x4 acc1[NT], acc2[NT];
  wg_mm<D>(A1, B1, K1, kNoMat, kNoMat, 0, lds, acc1);
  EpiD e = e1;
  e.x = nullptr;
  epilogue_d<D>(acc1, e);
  wg_mm<D>(A2, B2, K2, A3, B3, K2, lds, acc2);
  const int tid = threadIdx.x, w = tid >> 6, g = (tid & 63) >> 4, l16 = tid & 15;
  const int64_t lane = (int64_t)(16 * w + 4 * g) * D + l16;
  gcfloat* f1 = glb(e1.fx);
  gcfloat* f2 = glb(fx2);
  gfloat* x = glb(e1.x);
#pragma unroll
  for (int n0 = 0; n0 < NT; n0 += NH) {
    f32x4 a[NH], b[NH];
#pragma unroll
    for (int nt = 0; nt < NH; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[nt][i] = f1[lane + i * D + 16 * (n0 + nt)];
        b[nt][i] = f2[lane + i * D + 16 * (n0 + nt)];
      }
#pragma unroll
    for (int nt = 0; nt < NH; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[lane + i * D + 16 * (n0 + nt)] = (0.f + acc1[n0 + nt][i] * a[nt][i]) + acc2[n0 + nt][i] * b[nt][i];
  }
}

// out1 = A B1 and out2 = A B2, each with its own epilogue.
template <int D>
__device__ __attribute__((noinline)) void gemm_d2b(const Mat A, const Mat B1, const Mat B2, int K, float* lds,
                                                   const EpiD e1, const EpiD e2) {
  f32x4 acc1[D / 16], acc2[D / 16];
  wg_mm2b<D>(A, B1, B2, K, lds, acc1, acc2);
  epilogue_d<D>(acc1, e1);
  epilogue_d<D>(acc2, e2);
}

template <class In>
__device__ __forceinline__ float ld(const In* p, int64_t i) { return to_f32(p[i]); }

// ---------------------------------------------------------------------------
// Kernel 1: factors of one (chunk, head).
// ---------------------------------------------------------------------------
template <int D, class In>
__global__ __launch_bounds__(kThreads, 2) void bwd_prep(const In* __restrict__ q, const In* __restrict__ k,
                                                     const In* __restrict__ v, const float* __restrict__ log_alpha,
                                                     const In* __restrict__ beta, const In* __restrict__ grad_o,
                                                     const int32_t* __restrict__ cu, int N, int H,
                                                     const Win win) {
  using L = Ws<D>;
  __shared__ __align__(16) float lds[kGemmLds + 2 * C * C + C];
  float* sA = lds + kGemmLds;    // A
  float* sT = sA + C * C;        // T
  float* sBeta = sT + C * C;

  const int64_t item = blockIdx.x, slot = win.slot_lo + item / H;
  const int h = (int)(item % H);
  int n, len;
  int64_t t0;
  if (!decode_slot(cu, N, slot, n, t0, len)) return;
  float* B = win.blocks + item * L::FLOATS;
  const int tid = threadIdx.x;

  // the chunk's log decays, staged in LDS by the whole workgroup (rows past
  // the chunk's end read as zero).  Every load in this kernel reads a row
  // clamped into the chunk and selects zero afterwards, so that loads are
  // never conditional and can all be in flight together.
  float* sLa = lds;   // [C][D], overlaps the GEMM staging area (not yet in use)
#pragma unroll
  for (int it = 0; it < C * D / 4 / kThreads; ++it) {
    const int idx = tid + kThreads * it, r = idx / (D / 4), cq = idx % (D / 4);
    const f32x4 x = *reinterpret_cast<const f32x4*>(log_alpha + ((t0 + min(r, len - 1)) * H + h) * D + 4 * cq);
    *reinterpret_cast<f32x4*>(sLa + r * D + 4 * cq) = r < len ? x : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  // inputs: thread t owns key and value channel c = t % D for one of the
  // NG = 256 / D groups of rows (its cumulative decay, the key-side factors,
  // and the copies of v and dO)
  {
    constexpr int NG = kThreads / D, RG = C / NG;
    const int c = tid % D, grp = tid / D, r0 = grp * RG;
    // the cumulative decay and its exponentials in fp64: an fp32 running sum
    // over strong decays carries an absolute error that every factor
    // e^(G_r - G_s) would inherit as a relative one.  Every thread sums from
    // row 0 in the same order, so all groups see the same G.
    double gs = 0.0, a = 0.0, G = 0.0;
#pragma unroll 4
    for (int r = 0; r < C; ++r) {
      gs += (double)sLa[r * D + c];
      if (r == 31) a = gs;   // the anchor: mid-chunk
      if (r == r0 - 1) G = gs;
    }
    const double gC = gs;
    const double ea = exp(a), egc = exp(gC);
    if (grp == 0) B[L::GAM + c] = (float)egc;
#pragma unroll 1
    for (int x0 = 0; x0 < RG; x0 += 4) {
      float k8[4], q8[4], v8[4], o8[4];   // four rows' loads issued before any use
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t gi = ((t0 + min(r0 + x0 + i, len - 1)) * H + h) * D + c;
        k8[i] = ld(k, gi);
        q8[i] = ld(q, gi);
        v8[i] = ld(v, gi);
        o8[i] = ld(grad_o, gi);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + x0 + i;
        const bool in = r < len;
        const float kk = in ? k8[i] : 0.f, qq = in ? q8[i] : 0.f;
        G += (double)sLa[r * D + c];
        // one exponential per element; the other three factors follow from
        // it in fp64 (each product adds one fp64 rounding)
        const double xGa = exp(G - a), xaG = 1.0 / xGa;
        const float eGa = (float)xGa, eaG = (float)xaG, eG = (float)(xGa * ea), eC = (float)(egc * xaG / ea);
        const int64_t o = (int64_t)r * D + c;
        B[L::KX + o] = kk;
        B[L::QX + o] = qq;
        B[L::VX + o] = in ? v8[i] : 0.f;
        B[L::DOX + o] = in ? o8[i] : 0.f;
        B[L::EG + o] = eG;
        B[L::EC + o] = eC;
        B[L::EGA + o] = eGa;
        B[L::EAG + o] = eaG;
        B[L::KA + o] = kk * eGa;
        B[L::KB + o] = kk * eaG;
        B[L::QA + o] = qq * eGa;
        B[L::KG + o] = kk * eG;
        B[L::QG + o] = qq * eG;
        B[L::KC + o] = kk * eC;
      }
    }
  }
  if (tid < C) {
    const float b1 = ld(beta, (t0 + min(tid, len - 1)) * H + h);
    const float b = tid < len ? b1 : 0.f;
    B[L::BETA + tid] = b;
    sBeta[tid] = b;
  }
  // (wg_gemm starts with a barrier)

  // A = strict_lower(Ka Kb^T), Bq = lower(Qa Kb^T)
  wg_gemm<C>(Mat{B + L::KA, D, 1}, Mat{B + L::KB, 1, D}, D, lds, [=](int r, int s, float x) {
    x = s < r ? x : 0.f;
    glb(B)[L::A + r * C + s] = x;
    loc(sA)[r * C + s] = x;
  });
  wg_gemm<C>(Mat{B + L::QA, D, 1}, Mat{B + L::KB, 1, D}, D, lds,
             [=](int r, int s, float x) { glb(B)[L::BQ + r * C + s] = s <= r ? x : 0.f; });

  // T = (I + Diag(beta) A)^-1 = M^-1 (unit lower triangular), by 16 x 16
  // blocks: wave w inverts diagonal block w by substitution down its columns
  // (lane j walks column j; entries above the diagonal are stored as zeros,
  // so every sum runs without a test), then the blocks below the diagonal
  // follow level by level, T_ij = -T_ii sum_{j <= k < i} M_ik T_kj with
  // M_ik = Diag(beta) A_ik, each block by one wave.
  {
    const int w = tid >> 6, l = tid & 63;
    if (l < 16) {
      const int j = l, o = 16 * w;
      for (int r = 0; r < 16; ++r) {
        float a0 = 0.f, a1 = 0.f;
        for (int s = 0; s + 1 < r; s += 2) {
          a0 += sA[(o + r) * C + o + s] * sT[(o + s) * C + o + j];
          a1 += sA[(o + r) * C + o + s + 1] * sT[(o + s + 1) * C + o + j];
        }
        if (r & 1) a0 += sA[(o + r) * C + o + r - 1] * sT[(o + r - 1) * C + o + j];
        sT[(o + r) * C + o + j] = r == j ? 1.f : (r > j ? -sBeta[o + r] * (a0 + a1) : 0.f);
      }
    }
    // zeros above the diagonal blocks
    for (int idx = tid; idx < C * C; idx += kThreads) {
      const int r = idx / C, c = idx % C;
      if ((c >> 4) > (r >> 4)) sT[idx] = 0.f;
    }
    __syncthreads();
    float* sX = sLa;   // [4][16][16] scratch, one tile per wave (sLa is no longer needed)
    const int rr = l >> 2, c0 = (l & 3) * 4;
    for (int lev = 1; lev < 4; ++lev) {
      if (w < 4 - lev) {
        const int bj = w, bi = w + lev;
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        const float br = sBeta[16 * bi + rr];
        for (int bk = bj; bk < bi; ++bk)
          for (int s = 0; s < 16; ++s) {
            const float m = br * sA[(16 * bi + rr) * C + 16 * bk + s];
            const f32x4 t = *reinterpret_cast<const f32x4*>(sT + (16 * bk + s) * C + 16 * bj + c0);
#pragma unroll
            for (int q = 0; q < 4; ++q) x[q] += m * t[q];
          }
        *reinterpret_cast<f32x4*>(sX + w * 256 + rr * 16 + c0) = f32x4{x[0], x[1], x[2], x[3]};
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the tile is in LDS
        __builtin_amdgcn_wave_barrier();
        float t4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < 16; ++s) {
          const float tii = sT[(16 * bi + rr) * C + 16 * bi + s];
          const f32x4 xs = *reinterpret_cast<const f32x4*>(sX + w * 256 + s * 16 + c0);
#pragma unroll
          for (int q = 0; q < 4; ++q) t4[q] += tii * xs[q];
        }
        *reinterpret_cast<f32x4*>(sT + (16 * bi + rr) * C + 16 * bj + c0) = f32x4{-t4[0], -t4[1], -t4[2], -t4[3]};
      }
      __syncthreads();
    }
  }
  __syncthreads();
  for (int idx = tid; idx < C * C; idx += kThreads) {
    const float t = sT[idx];
    B[L::T + idx] = t;
    B[L::TB + idx] = t * sBeta[idx % C];
  }

  // W = Tb Kg, U = Tb V
  wg_gemm<D>(Mat{B + L::TB, C, 1}, Mat{B + L::KG, D, 1}, C, lds,
             [=](int r, int c, float x) { glb(B)[L::W + (int64_t)r * D + c] = x; });
  wg_gemm<D>(Mat{B + L::TB, C, 1}, Mat{B + L::VX, D, 1}, C, lds,
             [=](int r, int c, float x) { glb(B)[L::U + (int64_t)r * D + c] = x; });
}

// (sequence, head, 16-column slice) of a workgroup; same XCD-aware order as
// the forward state pass.  False when the workgroup has no pair.
template <int D>
__device__ __forceinline__ bool slice_of(int N, int H, int& n, int& h, int& vt) {
  constexpr int NV = D / 16;
  const int bid = blockIdx.x, xcd = bid & 7, rest = bid >> 3;
  vt = rest % NV;
  const int pair = (rest / NV) * 8 + xcd;
  if (pair >= N * H) return false;
  n = pair / H;
  h = pair % H;
  return true;
}

// The chunks [c_lo, c_hi) of a sequence whose slots lie in the window
// (c_hi == c_lo when there are none).
__device__ __forceinline__ void window_chunks(const Win& win, int64_t slot0, int nch, int& c_lo, int& c_hi) {
  c_lo = (int)max<int64_t>(0, win.slot_lo - slot0);
  c_hi = (int)max<int64_t>(c_lo, min<int64_t>(nch, win.slot_hi - slot0));
}

// ---------------------------------------------------------------------------
// Kernel 2: forward state pass over the window's chunks, storing S0 of every
// chunk (and of the first chunk after the window) and E of the window's.
// Wave w owns key tiles [KTW w, KTW (w+1)) of the slice and token tile w.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_fwd(const int32_t* __restrict__ cu, int N, int H,
                                                    const float* __restrict__ init, const Win win) {
  using L = Ws<D>;
  // LDS strides: W is read as the A operand over (token, key) pairs and Kc as
  // the A operand over (key, token) pairs; D + 2 and D + 16 make both reads
  // free of bank conflicts
  constexpr int KTW = D / 64, LW = D + 2, LK = D + 16;
  __shared__ __align__(16) float sW[C * LW];    // W  [token][key]
  __shared__ __align__(16) float sKc[C * LK];   // Kc [token][key]
  __shared__ __align__(16) float sS[D * 16];    // S slice [key][col]
  __shared__ __align__(16) float sE[C * 16];    // E slice [token][col]
  int n, h, vt;
  if (!slice_of<D>(N, H, n, h, vt)) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
  const int col = 16 * vt + l16;
  const int64_t bos = cu[n], eos = cu[n + 1];
  const int nch = (int)((eos - bos + C - 1) / C);
  const int64_t slot0 = bos / C + n;
  int c_lo, c_hi;
  window_chunks(win, slot0, nch, c_lo, c_hi);
  if (c_lo >= c_hi) return;
  // S0 of chunk c, [value column][key]
  auto s0_of = [&](int c) { return win.s0 + ((slot0 + c) * H + h) * (int64_t)D * D + (int64_t)col * D; };

  // the state entering the window: the initial state, or the one stored by
  // the window before
  f32x4 S[KTW];
#pragma unroll
  for (int kt = 0; kt < KTW; ++kt) {
    const int key0 = 16 * (w * KTW + kt) + 4 * g;
    if (c_lo > 0) S[kt] = *reinterpret_cast<const f32x4*>(s0_of(c_lo) + key0);
    else S[kt] = init ? *reinterpret_cast<const f32x4*>(init + (((int64_t)n * H + h) * D + col) * D + key0)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto block = [&](int c) { return win.blocks + ((slot0 + c - win.slot_lo) * H + h) * L::FLOATS; };
  // the next chunk's operands are loaded into registers while this chunk is
  // computed: W and Kc (NQ quads each per thread), this lane's U and e^gC,
  // in two parts issued during the two products, so that the vector memory
  // path works while the matrix cores do
  constexpr int NQ = C * D / 4 / kThreads;
  f32x4 pw[NQ], pk[NQ], pg[KTW];
  float pu[4];
  auto fetch = [&](int c, int part) {
    const float* B = block(c);
    if (part == 0) {
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int idx = tid + kThreads * i, r = idx / (D / 4), cq = idx % (D / 4);
        pw[i] = *reinterpret_cast<const f32x4*>(B + L::W + (int64_t)r * D + 4 * cq);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pu[i] = B[L::U + (int64_t)(16 * w + 4 * g + i) * D + col];
    } else {
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int idx = tid + kThreads * i, r = idx / (D / 4), cq = idx % (D / 4);
        pk[i] = *reinterpret_cast<const f32x4*>(B + L::KC + (int64_t)r * D + 4 * cq);
      }
#pragma unroll
      for (int kt = 0; kt < KTW; ++kt)
        pg[kt] = *reinterpret_cast<const f32x4*>(B + L::GAM + 16 * (w * KTW + kt) + 4 * g);
    }
  };
  if (c_lo < c_hi) {
    fetch(c_lo, 0);
    fetch(c_lo, 1);
  }
  for (int c = c_lo; c < c_hi; ++c) {
    float* B = block(c);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int idx = tid + kThreads * i, r = idx / (D / 4), cq = idx % (D / 4);
      *reinterpret_cast<float2*>(sW + r * LW + 4 * cq) = float2{pw[i][0], pw[i][1]};
      *reinterpret_cast<float2*>(sW + r * LW + 4 * cq + 2) = float2{pw[i][2], pw[i][3]};
      *reinterpret_cast<f32x4*>(sKc + r * LK + 4 * cq) = pk[i];
    }
    float u[4];
    f32x4 gam[KTW];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = pu[i];
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) gam[kt] = pg[kt];
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int key0 = 16 * (w * KTW + kt) + 4 * g;
      *reinterpret_cast<f32x4*>(s0_of(c) + key0) = S[kt];
#pragma unroll
      for (int i = 0; i < 4; ++i) sS[(key0 + i) * 16 + l16] = S[kt][i];
    }
    __syncthreads();
    if (c + 1 < c_hi) fetch(c + 1, 0);
    // E = U - W S for token tile w
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 4) acc = mfma4(sW[(16 * w + l16) * LW + k0 + g], sS[(k0 + g) * 16 + l16], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g + i;
      const float e = u[i] - acc[i];
      B[L::E + (int64_t)r * D + col] = e;
      sE[r * 16 + l16] = e;
    }
    __syncthreads();
    if (c + 1 < c_hi) fetch(c + 1, 1);
    // S <- Diag(gamma) S + Kc^T E
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int key0 = 16 * (w * KTW + kt);
      S[kt] *= gam[kt];
#pragma unroll
      for (int t = 0; t < C; t += 4) S[kt] = mfma4(sKc[(t + g) * LK + key0 + l16], sE[(t + g) * 16 + l16], S[kt]);
    }
    __syncthreads();
  }
  // the state entering the next window's first chunk of this sequence
  if (c_hi < nch) {
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt)
      *reinterpret_cast<f32x4*>(s0_of(c_hi) + 16 * (w * KTW + kt) + 4 * g) = S[kt];
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: reverse pass over the window's chunks for dL/dS; stores dS_end
// and dE of each, hands dL/dS to the window before (carry) or, at the
// sequence's first chunk, writes dL/dS_0.  A sequence without chunks is
// handled by the first window (the last reverse pass to run).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dstate(const int32_t* __restrict__ cu, int N, int H,
                                                       const float* grad_final, float* grad_init, const Win win) {
  // grad_init may be the grad_final buffer (in-place): each element is read
  // before the same thread writes it, so the two are not declared restrict
  using L = Ws<D>;
  // LDS strides chosen so that every MFMA operand read is conflict-free:
  // Bq is read over (token, s) pairs, Kc over (token, key), Qg and W over
  // (key, token)
  constexpr int KTW = D / 64, LC = C + 16, LK = D + 16, LR = D + 2;
  __shared__ __align__(16) float sBq[C * LC];   // Bq [s][token]
  __shared__ __align__(16) float sKc[C * LR];   // Kc [token][key]
  __shared__ __align__(16) float sQg[C * LK];   // Qg [token][key]
  __shared__ __align__(16) float sW[C * LK];    // W  [token][key]
  __shared__ __align__(16) float sdO[C * 16];
  __shared__ __align__(16) float sdS[D * 16];
  __shared__ __align__(16) float snE[C * 16];
  int n, h, vt;
  if (!slice_of<D>(N, H, n, h, vt)) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
  const int col = 16 * vt + l16;
  const int64_t bos = cu[n], eos = cu[n + 1];
  const int nch = (int)((eos - bos + C - 1) / C);
  const int64_t slot0 = bos / C + n;
  const int64_t sbase = (((int64_t)n * H + h) * D + col) * D;
  int c_lo, c_hi;
  window_chunks(win, slot0, nch, c_lo, c_hi);
  if (nch > 0 ? c_lo >= c_hi : win.slot_lo != 0) return;

  // dL/dS after the window: the upstream final-state gradient, or what the
  // window after handed over
  f32x4 dS[KTW];
#pragma unroll
  for (int kt = 0; kt < KTW; ++kt) {
    const int key0 = 16 * (w * KTW + kt) + 4 * g;
    if (c_hi < nch) dS[kt] = *reinterpret_cast<const f32x4*>(win.carry + sbase + key0);
    else dS[kt] = grad_final ? *reinterpret_cast<const f32x4*>(grad_final + sbase + key0) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto block = [&](int c) { return win.blocks + ((slot0 + c - win.slot_lo) * H + h) * L::FLOATS; };
  // the previous chunk's operands are loaded into registers while this one
  // is computed, in two parts issued during the two products, so that the
  // vector memory path works while the matrix cores do
  constexpr int NQ = C * D / 4 / kThreads, NB = C * C / 4 / kThreads;
  f32x4 pb[NB], pk[NQ], pq[NQ], pw[NQ], po, pg[KTW];
  auto fetch = [&](int c, int part) {
    const float* B = block(c);
    if (part == 0) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int idx = tid + kThreads * i, s = idx / (C / 4), tq = idx % (C / 4);
        pb[i] = *reinterpret_cast<const f32x4*>(B + L::BQ + s * C + 4 * tq);
      }
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int idx = tid + kThreads * i, r = idx / (D / 4), cq = idx % (D / 4);
        pk[i] = *reinterpret_cast<const f32x4*>(B + L::KC + (int64_t)r * D + 4 * cq);
      }
      po = *reinterpret_cast<const f32x4*>(B + L::DOX + (int64_t)(tid >> 2) * D + 16 * vt + 4 * (tid & 3));
    } else {
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int idx = tid + kThreads * i, r = idx / (D / 4), cq = idx % (D / 4);
        pq[i] = *reinterpret_cast<const f32x4*>(B + L::QG + (int64_t)r * D + 4 * cq);
        pw[i] = *reinterpret_cast<const f32x4*>(B + L::W + (int64_t)r * D + 4 * cq);
      }
#pragma unroll
      for (int kt = 0; kt < KTW; ++kt)
        pg[kt] = *reinterpret_cast<const f32x4*>(B + L::GAM + 16 * (w * KTW + kt) + 4 * g);
    }
  };
  if (c_hi > c_lo) {
    fetch(c_hi - 1, 0);
    fetch(c_hi - 1, 1);
  }
  for (int c = c_hi - 1; c >= c_lo; --c) {
    float* B = block(c);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int idx = tid + kThreads * i, s = idx / (C / 4), tq = idx % (C / 4);
      *reinterpret_cast<f32x4*>(sBq + s * LC + 4 * tq) = pb[i];
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int idx = tid + kThreads * i, r = idx / (D / 4), cq = idx % (D / 4);
      *reinterpret_cast<float2*>(sKc + r * LR + 4 * cq) = float2{pk[i][0], pk[i][1]};
      *reinterpret_cast<float2*>(sKc + r * LR + 4 * cq + 2) = float2{pk[i][2], pk[i][3]};
      *reinterpret_cast<f32x4*>(sQg + r * LK + 4 * cq) = pq[i];
      *reinterpret_cast<f32x4*>(sW + r * LK + 4 * cq) = pw[i];
    }
    *reinterpret_cast<f32x4*>(sdO + (tid >> 2) * 16 + 4 * (tid & 3)) = po;
    f32x4 gam[KTW];
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) gam[kt] = pg[kt];
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int key0 = 16 * (w * KTW + kt) + 4 * g;
      *reinterpret_cast<f32x4*>(B + L::DS + (int64_t)col * D + key0) = dS[kt];
#pragma unroll
      for (int i = 0; i < 4; ++i) sdS[(key0 + i) * 16 + l16] = dS[kt][i];
    }
    __syncthreads();
    if (c > c_lo) fetch(c - 1, 0);
    // dE = Bq^T dO + Kc dS for token tile w
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int s = 0; s < C; s += 4) acc = mfma4(sBq[(s + g) * LC + 16 * w + l16], sdO[(s + g) * 16 + l16], acc);
#pragma unroll 16
    for (int k0 = 0; k0 < D; k0 += 4) acc = mfma4(sKc[(16 * w + l16) * LR + k0 + g], sdS[(k0 + g) * 16 + l16], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g + i;
      B[L::DE + (int64_t)r * D + col] = acc[i];
      snE[r * 16 + l16] = -acc[i];
    }
    __syncthreads();
    if (c > c_lo) fetch(c - 1, 1);
    // dS <- Diag(gamma) dS + Qg^T dO - W^T dE
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int key0 = 16 * (w * KTW + kt);
      dS[kt] *= gam[kt];
#pragma unroll 8
      for (int t = 0; t < C; t += 4) {
        dS[kt] = mfma4(sQg[(t + g) * LK + key0 + l16], sdO[(t + g) * 16 + l16], dS[kt]);
        dS[kt] = mfma4(sW[(t + g) * LK + key0 + l16], snE[(t + g) * 16 + l16], dS[kt]);
      }
    }
    __syncthreads();
  }
  float* dst = c_lo > 0 ? win.carry : grad_init;
  if (dst) {
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int key0 = 16 * (w * KTW + kt) + 4 * g;
      *reinterpret_cast<f32x4*>(dst + sbase + key0) = dS[kt];
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 4: per-(chunk, head) gradients.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_grad(const int32_t* __restrict__ cu, int N, int H,
                                                     const Win win, float* __restrict__ gq,
                                                     float* __restrict__ gk, float* __restrict__ gv,
                                                     float* __restrict__ gla, float* __restrict__ gbeta) {
  using L = Ws<D>;
  __shared__ __align__(16) float lds[kGemmLds3 > kGemmLds2 ? kGemmLds3 : kGemmLds2];
  __shared__ float sPV[C], sRK[C];    // rowsum(P o V), rowsum(R o Kg)
  __shared__ double sKc[16 * D];      // partial colsums of dKc o Kc
  const int64_t item = blockIdx.x, slot = win.slot_lo + item / H;
  const int h = (int)(item % H);
  int n, len;
  int64_t t0;
  if (!decode_slot(cu, N, slot, n, t0, len)) return;
  float* B = win.blocks + item * L::FLOATS;
  const float* S0 = win.s0 + (slot * H + h) * (int64_t)D * D;   // [value column][key]
  const float* beta = B + L::BETA;
  auto at = [&](int64_t base, int r, int c) -> float& { return B[base + (int64_t)r * D + c]; };
  auto M = [&](int64_t base, int rs, int cs) { return Mat{B + base, rs, cs}; };
  auto F = [&](int64_t base) { return B + base; };

  // dBq = lower(dO E^T), kept as its strict lower part and its diagonal:
  // Bq[r][r] = q_r . k_r carries no decay, so its terms would enter dG twice
  // with opposite signs; they go straight to dq and dk instead
  wg_gemm<C>(M(L::DOX, D, 1), M(L::E, 1, D), D, lds, [=](int r, int s, float x) {
    glb(B)[L::DBQ + r * C + s] = s < r ? x : 0.f;
    if (s == r) glb(B)[L::DBQD + r] = x;
  });
  {  // dQg = dO S0^T: dQ = dQg e^G; dW = -dE S0^T
    EpiD e1, e2;
    e1.x = F(L::DQ); e1.fx = F(L::EG);
    e2.store = F(L::DW); e2.store_scale = -1.f;
    gemm_d2<D>(M(L::DOX, D, 1), M(L::DE, D, 1), Mat{S0, D, 1}, D, lds, e1, e2);
  }
  {  // P = T^T dE: dV = Diag(beta) P; rowsum(P o V) for dbeta;
     // R = T^T dW: dKg = Diag(beta) R: dKp = dKg e^G; rowsum(R o Kg) for dbeta
    EpiD e1, e2;
    e1.out = gv + (t0 * H + h) * D; e1.out_rs = (int64_t)H * D; e1.len = len; e1.beta = beta;
    e1.rowsum = sPV; e1.rf = F(L::VX);
    e2.x = F(L::DKP); e2.fx = F(L::EG);
    e2.rowsum = sRK; e2.rf = F(L::KG);
    e2.row_beta = true; e2.beta = beta;
    gemm_d2b<D>(M(L::T, 1, C), M(L::DE, D, 1), M(L::DW, D, 1), C, lds, e1, e2);
  }
  // dT = dE (Diag(beta) V)^T + dW (Diag(beta) Kg)^T  (beta of the column)
  {
    f32x4 a[C / 16];
    wg_mm<C>(M(L::DE, D, 1), M(L::VX, 1, D), D, M(L::DW, D, 1), M(L::KG, 1, D), D, lds, a);
    const int w = threadIdx.x >> 6, g = (threadIdx.x & 63) >> 4, l16 = threadIdx.x & 15;
#pragma unroll
    for (int nt = 0; nt < C / 16; ++nt) {
      const float bc = beta[16 * nt + l16];
#pragma unroll
      for (int i = 0; i < 4; ++i) B[L::DT + (16 * w + 4 * g + i) * C + 16 * nt + l16] = bc * a[nt][i];
    }
  }
  // X = dT T^T; dM = -T^T X: dA = strict_lower(Diag(beta) dM), dMA = strict_lower(dM) o A
  wg_gemm<C>(M(L::DT, C, 1), M(L::T, 1, C), C, lds, [=](int r, int s, float x) { glb(B)[L::X + r * C + s] = x; });
  wg_gemm<C>(M(L::T, 1, C), M(L::X, C, 1), C, lds, [=](int r, int s, float x) {
    const float dm = -x;
    glb(B)[L::DA + r * C + s] = s < r ? glb(beta)[r] * dm : 0.f;
    glb(B)[L::DMA + r * C + s] = s < r ? dm * glb(B)[L::A + r * C + s] : 0.f;
  });
  // dQa = dBs Kb: dQ += dQa e^(G-a); dKa = dA Kb: dKp += dKa e^(G-a)
  gemm_d2_addf<D>(M(L::DBQ, C, 1), M(L::DA, C, 1), M(L::KB, D, 1), C, lds, F(L::DQ), F(L::DKP), F(L::EGA));
  {  // dKc = E dS_end^T, colsum(dKc o Kc) for dgC; dKb = dA^T Ka + dBs^T Qa;
     // dKm = dKc e^(gC-G) + dKb e^(a-G)
    EpiD e;
    e.x = F(L::DKM); e.fx = F(L::EC);
    e.colsum = sKc; e.cf = F(L::KC);
    gemm_d_sum2<D>(M(L::E, D, 1), M(L::DS, D, 1), D, M(L::DA, 1, C), M(L::KA, D, 1), M(L::DBQ, 1, C),
                   M(L::QA, D, 1), C, F(L::EAG), lds, e);
  }
  __syncthreads();

  // element-wise assembly.  Thread t owns key channel c = t % D and one of
  // NG = 256 / D groups of rows; group partial sums meet in LDS (fixed order).
  constexpr int NG = kThreads / D, RG = C / NG, JG = D / NG;
  double* sRed = reinterpret_cast<double*>(lds);   // [NG][D]: partials, then group totals
  double* sDgc = sRed + NG * D;                     // [D]
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int c = tid % D, grp = tid / D;
  {
    double dgam = 0.0, dkc = 0.0;
#pragma unroll 16
    for (int j = grp * JG; j < (grp + 1) * JG; ++j)
      dgam += (double)B[L::DS + (int64_t)j * D + c] * (double)S0[(int64_t)j * D + c];
    for (int x = grp * (16 / NG); x < (grp + 1) * (16 / NG); ++x) dkc += sKc[x * D + c];
    // partial of dgC = rowsum(dS_end o S0) gamma + colsum(dKc o Kc)
    sRed[grp * D + c] = dgam * (double)B[L::GAM + c] + dkc;
  }
  __syncthreads();
  if (tid < D) {
    double t = 0.0;
    for (int x = 0; x < NG; ++x) t += sRed[x * D + tid];
    sDgc[tid] = t;
  }
  // d log_alpha[r] = sum_{s >= r} dG[s] + dgC: each group sums its own rows
  // bottom-up, then adds the totals of the groups below it
  double suf[RG];
  {
    double acc2 = 0.0;
#pragma unroll
    for (int x = RG - 1; x >= 0; --x) {
      const int r = grp * RG + x;
      acc2 += (double)at(L::KX, r, c) * ((double)at(L::DKP, r, c) - (double)at(L::DKM, r, c)) +
              (double)at(L::QX, r, c) * (double)at(L::DQ, r, c);
      suf[x] = acc2;
    }
    __syncthreads();   // sRed partials consumed
    sRed[grp * D + c] = acc2;
  }
  __syncthreads();
  {
    double later = sDgc[c];
    for (int x = grp + 1; x < NG; ++x) later += sRed[x * D + c];
#pragma unroll
    for (int x = 0; x < RG; ++x) {
      const int r = grp * RG + x;
      const float dd = B[L::DBQD + r];
      const float gqv = at(L::DQ, r, c) + dd * at(L::KX, r, c);
      const float gkv = at(L::DKP, r, c) + at(L::DKM, r, c) + dd * at(L::QX, r, c);
      if (r < len) {
        const int64_t o = ((t0 + r) * H + h) * D + c;
        gla[o] = (float)(suf[x] + later);
        gq[o] = gqv;
        gk[o] = gkv;
      }
    }
  }
  // dbeta = rowsum(P o V) + rowsum(R o Kg) + rowsum(strict_lower(dM) o A):
  // wave w reduces the last term over rows [16 w, 16 w + 16), its lanes
  // across columns
#pragma unroll 4
  for (int rr = 0; rr < 16; ++rr) {
    const int r = 16 * (tid >> 6) + rr;
    float part = B[L::DMA + r * C + l];   // strictly lower: zero for l >= r
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) part += __shfl_xor(part, m);
    if (l == 0 && r < len) gbeta[(t0 + r) * H + h] = sPV[r] + sRK[r] + part;
  }
}

// Window budget: at most 512 chunk slots and 8 GiB of blocks per window (the
// 8K workload at H = 32, 130 slots of 4.3 GB, is one window).
constexpr int64_t kWindowSlots = 512;
constexpr size_t kWindowBytes = (size_t)8 << 30;

template <int D>
static int64_t window_slots(int64_t slots, int H) {
  const int64_t by_bytes = (int64_t)(kWindowBytes / ((size_t)H * Ws<D>::FLOATS * sizeof(float)));
  return std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(slots, kWindowSlots), by_bytes));
}

// Workspace: the window's blocks, S0 of every chunk slot, the carry.
template <int D>
static size_t workspace_bytes_t(int32_t N, int64_t slots, int H) {
  return ((size_t)window_slots<D>(slots, H) * H * Ws<D>::FLOATS + (size_t)slots * H * D * D +
          (size_t)N * H * D * D) * sizeof(float);
}

template <int D, class In>
static hipError_t launch_t(const BackwardArgs& A, hipStream_t stream) {
  const int64_t slots = prefill_num_slots(A.num_seqs, A.total_tokens);
  const int H = A.num_heads;
  const int64_t wsl = window_slots<D>(slots, H);
  float* base = (float*)A.workspace;
  Win win{0, 0, base, nullptr, nullptr};
  if (base) {
    win.s0 = base + wsl * H * Ws<D>::FLOATS;
    win.carry = win.s0 + slots * H * (int64_t)D * D;
  }
  const int64_t pairs = (int64_t)A.num_seqs * H;
  const unsigned blocks = (unsigned)(((pairs + 7) / 8) * 8 * (D / 16));
  auto dstate = [&]() {
    hipLaunchKernelGGL((bwd_dstate<D>), dim3(blocks), dim3(kThreads), 0, stream, A.cu_seqlens, A.num_seqs, H,
                       A.grad_final_state, A.grad_init_state, win);
    return hipGetLastError();
  };
  if (A.total_tokens == 0) return dstate();   // no chunks: dL/dS_0 = dL/dS_T
  auto prep_fwd = [&]() {
    const unsigned items = (unsigned)((win.slot_hi - win.slot_lo) * H);
    hipLaunchKernelGGL((bwd_prep<D, In>), dim3(items), dim3(kThreads), 0, stream, (const In*)A.q, (const In*)A.k,
                       (const In*)A.v, A.log_alpha, (const In*)A.beta, (const In*)A.grad_o, A.cu_seqlens, A.num_seqs,
                       H, win);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_fwd<D>), dim3(blocks), dim3(kThreads), 0, stream, A.cu_seqlens, A.num_seqs, H,
                       A.init_state, win);
    return hipGetLastError();
  };
  const int64_t nwin = (slots + wsl - 1) / wsl;
  auto select = [&](int64_t w) {
    win.slot_lo = w * wsl;
    win.slot_hi = std::min<int64_t>(slots, win.slot_lo + wsl);
  };
  hipError_t e = hipSuccess;
  for (int64_t w = 0; w < nwin && e == hipSuccess; ++w) {   // forward sweep: S0 of every chunk
    select(w);
    e = prep_fwd();
  }
  for (int64_t w = nwin - 1; w >= 0 && e == hipSuccess; --w) {   // reverse sweep
    select(w);
    if (w != nwin - 1) e = prep_fwd();   // the last window's blocks are still in place
    if (e == hipSuccess) e = dstate();
    if (e == hipSuccess) {
      hipLaunchKernelGGL((bwd_grad<D>), dim3((unsigned)((win.slot_hi - win.slot_lo) * H)), dim3(kThreads), 0, stream,
                         A.cu_seqlens, A.num_seqs, H, win, A.grad_q, A.grad_k, A.grad_v, A.grad_log_alpha,
                         A.grad_beta);
      e = hipGetLastError();
    }
  }
  return e;
}

}  // namespace bwd

size_t backward_workspace_bytes(int32_t num_seqs, int64_t slots, int num_heads, int d) {
  return d == 128 ? bwd::workspace_bytes_t<128>(num_seqs, slots, num_heads)
                  : bwd::workspace_bytes_t<64>(num_seqs, slots, num_heads);
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.bf16 ? bwd::launch_t<128, __bf16>(a, stream) : bwd::launch_t<128, float>(a, stream);
  return a.bf16 ? bwd::launch_t<64, __bf16>(a, stream) : bwd::launch_t<64, float>(a, stream);
}

}  // namespace kda
