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
// Everything per chunk lives in a per-(chunk, head) block of the workspace.
#include "kda_launch.h"
#include "kda_prefill_common.h"

namespace kda {
namespace bwd {

constexpr int C = kChunk;

// Per-(chunk, head) workspace block, in floats.  Row-major [rows][cols];
// S0 and DS are stored like the states: [value column][key].  EG, EC, EGA,
// EAG hold e^G, e^(gC-G), e^(G-a), e^(a-G) and GAM e^gC, each evaluated in
// fp64 and rounded once; DG (the gradient of the cumulative decay) is
// accumulated in fp64.
template <int D>
struct Ws {
  static constexpr int64_t CD = (int64_t)C * D, CC = (int64_t)C * C, DD = (int64_t)D * D;
  static constexpr int64_t KX = 0, QX = CD, VX = 2 * CD, DOX = 3 * CD, KA = 4 * CD, KB = 5 * CD, QA = 6 * CD,
                           KG = 7 * CD, QG = 8 * CD, KC = 9 * CD, EG = 10 * CD, EC = 11 * CD, EGA = 12 * CD,
                           EAG = 13 * CD, W = 14 * CD, U = 15 * CD, E = 16 * CD, DE = 17 * CD, DQ = 18 * CD,
                           DK = 19 * CD, DKC = 20 * CD, DW = 21 * CD, P = 22 * CD, R = 23 * CD;
  static constexpr int64_t DG = 24 * CD;   // fp64 [C][D], two floats per element
  static constexpr int64_t A = 26 * CD, BQ = A + CC, T = BQ + CC, TB = T + CC, DBQ = TB + CC, DT = DBQ + CC,
                           X = DT + CC, DA = X + CC, DMA = DA + CC;
  static constexpr int64_t S0 = DMA + CC, DS = S0 + DD;
  static constexpr int64_t BETA = DS + DD, DBQD = BETA + C, GAM = DBQD + C;
  static constexpr int64_t FLOATS = GAM + D;
  static_assert(FLOATS % 4 == 0, "blocks stay 16-byte aligned");
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

// out (64 x N) = A (64 x Kd) B (Kd x N) by the whole workgroup (wave w owns
// output rows [16 w, 16 w + 16)); Kd a multiple of 32.  Panels of 32
// reduction indices are staged in LDS, reduction-index major, so that every
// MFMA operand read is conflict-free.  epi(row, col, value) is called once
// per output element, by the lane that owns it.  Begins and ends with a
// barrier, so the epilogue's writes are visible to the next call.
constexpr int kGemmLds = 32 * 80 + 32 * 144;   // floats, for N <= 128

template <int N, class Epi>
__device__ __attribute__((noinline)) void wg_gemm(const Mat A, const Mat B, int Kd, float* lds, Epi epi) {
  constexpr int LA = 80, LB = N + 16;
  float* sA = lds;
  float* sB = lds + 32 * LA;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
  f32x4 acc[N / 16];
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  for (int k0 = 0; k0 < Kd; k0 += 32) {
    if (A.cs == 1) {   // reduction index contiguous in memory
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int idx = tid + 256 * it, r = idx & 63, kq = idx >> 6;
        const f32x4 x = *reinterpret_cast<const f32x4*>(A.p + (int64_t)r * A.rs + k0 + 4 * kq);
#pragma unroll
        for (int i = 0; i < 4; ++i) sA[(4 * kq + i) * LA + r] = x[i];
      }
    } else {           // row index contiguous
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int idx = tid + 256 * it, rq = idx & 15, k = idx >> 4;
        *reinterpret_cast<f32x4*>(sA + k * LA + 4 * rq) =
            *reinterpret_cast<const f32x4*>(A.p + (int64_t)(k0 + k) * A.cs + 4 * rq);
      }
    }
    if (B.cs == 1) {   // column index contiguous
      for (int idx = tid; idx < 8 * N; idx += 256) {
        const int nq = idx % (N / 4), k = idx / (N / 4);
        *reinterpret_cast<f32x4*>(sB + k * LB + 4 * nq) =
            *reinterpret_cast<const f32x4*>(B.p + (int64_t)(k0 + k) * B.rs + 4 * nq);
      }
    } else {           // reduction index contiguous
      for (int idx = tid; idx < 8 * N; idx += 256) {
        const int n = idx % N, kq = idx / N;
        const f32x4 x = *reinterpret_cast<const f32x4*>(B.p + (int64_t)n * B.cs + k0 + 4 * kq);
#pragma unroll
        for (int i = 0; i < 4; ++i) sB[(4 * kq + i) * LB + n] = x[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      const float a = sA[(kk + g) * LA + 16 * w + l16];
#pragma unroll
      for (int nt = 0; nt < N / 16; ++nt) acc[nt] = mfma4(a, sB[(kk + g) * LB + 16 * nt + l16], acc[nt]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) epi(16 * w + 4 * g + i, 16 * nt + l16, acc[nt][i]);
  __syncthreads();
}

template <class In>
__device__ __forceinline__ float ld(const In* p, int64_t i) { return to_f32(p[i]); }

// ---------------------------------------------------------------------------
// Kernel 1: factors of one (chunk, head).
// ---------------------------------------------------------------------------
template <int D, class In>
__global__ __launch_bounds__(kThreads) void bwd_prep(const In* __restrict__ q, const In* __restrict__ k,
                                                     const In* __restrict__ v, const float* __restrict__ log_alpha,
                                                     const In* __restrict__ beta, const In* __restrict__ grad_o,
                                                     const int32_t* __restrict__ cu, int N, int H,
                                                     float* __restrict__ ws) {
  using L = Ws<D>;
  __shared__ __align__(16) float lds[kGemmLds + 2 * C * C + C];
  float* sA = lds + kGemmLds;    // A
  float* sT = sA + C * C;        // T
  float* sBeta = sT + C * C;

  const int64_t item = blockIdx.x, slot = item / H;
  const int h = (int)(item % H);
  int n, len;
  int64_t t0;
  if (!decode_slot(cu, N, slot, n, t0, len)) return;
  float* B = ws + item * L::FLOATS;
  const int tid = threadIdx.x;

  // inputs: thread c < D owns key channel c (its cumulative decay and the
  // key-side factors); thread D + c copies value channel c of v and dO
  if (tid < D) {
    const int c = tid;
    // the cumulative decay and its exponentials in fp64: an fp32 running sum
    // over strong decays carries an absolute error that every factor
    // e^(G_r - G_s) would inherit as a relative one
    double gs = 0.0, a = 0.0;
    for (int r = 0; r < C; ++r) {
      gs += r < len ? (double)log_alpha[((t0 + r) * H + h) * D + c] : 0.0;
      if (r == 31) a = gs;   // the anchor: mid-chunk
    }
    const double gC = gs;
    B[L::GAM + c] = (float)exp(gC);
    double G = 0.0;   // the same sums again, in the same order
    for (int r = 0; r < C; ++r) {
      const int64_t gi = ((t0 + r) * H + h) * D + c;
      const float kk = r < len ? ld(k, gi) : 0.f, qq = r < len ? ld(q, gi) : 0.f;
      G += r < len ? (double)log_alpha[gi] : 0.0;
      const float eGa = (float)exp(G - a), eaG = (float)exp(a - G), eG = (float)exp(G), eC = (float)exp(gC - G);
      const int64_t o = (int64_t)r * D + c;
      B[L::KX + o] = kk;
      B[L::QX + o] = qq;
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
  } else if (tid < 2 * D) {
    const int c = tid - D;
    for (int r = 0; r < C; ++r) {
      const int64_t gi = ((t0 + r) * H + h) * D + c;
      B[L::VX + (int64_t)r * D + c] = r < len ? ld(v, gi) : 0.f;
      B[L::DOX + (int64_t)r * D + c] = r < len ? ld(grad_o, gi) : 0.f;
    }
  }
  if (tid < C) {
    const float b = tid < len ? ld(beta, (t0 + tid) * H + h) : 0.f;
    B[L::BETA + tid] = b;
    sBeta[tid] = b;
  }
  // (wg_gemm starts with a barrier)

  // A = strict_lower(Ka Kb^T), Bq = lower(Qa Kb^T)
  wg_gemm<C>(Mat{B + L::KA, D, 1}, Mat{B + L::KB, 1, D}, D, lds, [&](int r, int s, float x) {
    x = s < r ? x : 0.f;
    B[L::A + r * C + s] = x;
    sA[r * C + s] = x;
  });
  wg_gemm<C>(Mat{B + L::QA, D, 1}, Mat{B + L::KB, 1, D}, D, lds,
             [&](int r, int s, float x) { B[L::BQ + r * C + s] = s <= r ? x : 0.f; });

  // T = (I + Diag(beta) A)^-1: columns are independent; lane j of wave 0
  // walks down column j (T[r][j] = -beta_r sum_{j <= s < r} A[r][s] T[s][j])
  if (tid < C) {
    const int j = tid;
    for (int r = 0; r < C; ++r) {
      float acc = 0.f;
      for (int s = 0; s < r; ++s) acc += s >= j ? sA[r * C + s] * sT[s * C + j] : 0.f;
      sT[r * C + j] = r == j ? 1.f : (r > j ? -sBeta[r] * acc : 0.f);
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
             [&](int r, int c, float x) { B[L::W + (int64_t)r * D + c] = x; });
  wg_gemm<D>(Mat{B + L::TB, C, 1}, Mat{B + L::VX, D, 1}, C, lds,
             [&](int r, int c, float x) { B[L::U + (int64_t)r * D + c] = x; });
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

// ---------------------------------------------------------------------------
// Kernel 2: forward state pass, storing S0 and E of every chunk.
// Wave w owns key tiles [KTW w, KTW (w+1)) of the slice and token tile w.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_fwd(const int32_t* __restrict__ cu, int N, int H,
                                                    const float* __restrict__ init, float* __restrict__ ws) {
  using L = Ws<D>;
  constexpr int KTW = D / 64, LW = C + 16, LK = D + 16;
  __shared__ __align__(16) float sWt[D * LW];   // W^T  [key][token]
  __shared__ __align__(16) float sKc[C * LK];   // Kc   [token][key]
  __shared__ __align__(16) float sS[D * 16];    // S slice [key][col]
  __shared__ __align__(16) float sE[C * 16];    // E slice [token][col]
  int n, h, vt;
  if (!slice_of<D>(N, H, n, h, vt)) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
  const int col = 16 * vt + l16;
  const int64_t bos = cu[n], eos = cu[n + 1];
  const int nch = (int)((eos - bos + C - 1) / C);
  const int64_t slot0 = bos / C + n;

  f32x4 S[KTW];
#pragma unroll
  for (int kt = 0; kt < KTW; ++kt) {
    const int key0 = 16 * (w * KTW + kt) + 4 * g;
    S[kt] = init ? *reinterpret_cast<const f32x4*>(init + (((int64_t)n * H + h) * D + col) * D + key0)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int c = 0; c < nch; ++c) {
    float* B = ws + ((slot0 + c) * H + h) * L::FLOATS;
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int key0 = 16 * (w * KTW + kt) + 4 * g;
      *reinterpret_cast<f32x4*>(B + L::S0 + (int64_t)col * D + key0) = S[kt];
#pragma unroll
      for (int i = 0; i < 4; ++i) sS[(key0 + i) * 16 + l16] = S[kt][i];
    }
    for (int idx = tid; idx < C * D / 4; idx += kThreads) {
      const int r = idx / (D / 4), cq = idx % (D / 4);
      const f32x4 x = *reinterpret_cast<const f32x4*>(B + L::W + (int64_t)r * D + 4 * cq);
#pragma unroll
      for (int i = 0; i < 4; ++i) sWt[(4 * cq + i) * LW + r] = x[i];
      *reinterpret_cast<f32x4*>(sKc + r * LK + 4 * cq) = *reinterpret_cast<const f32x4*>(B + L::KC + (int64_t)r * D + 4 * cq);
    }
    __syncthreads();
    // E = U - W S for token tile w
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int k0 = 0; k0 < D; k0 += 4) acc = mfma4(sWt[(k0 + g) * LW + 16 * w + l16], sS[(k0 + g) * 16 + l16], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g + i;
      const float e = B[L::U + (int64_t)r * D + col] - acc[i];
      B[L::E + (int64_t)r * D + col] = e;
      sE[r * 16 + l16] = e;
    }
    __syncthreads();
    // S <- Diag(gamma) S + Kc^T E
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int key0 = 16 * (w * KTW + kt);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[kt][i] *= B[L::GAM + key0 + 4 * g + i];
#pragma unroll 4
      for (int t = 0; t < C; t += 4) S[kt] = mfma4(sKc[(t + g) * LK + key0 + l16], sE[(t + g) * 16 + l16], S[kt]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: reverse pass over the chunks for dL/dS; stores dS_end and dE of
// every chunk and dL/dS_0 of the sequence.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dstate(const int32_t* __restrict__ cu, int N, int H,
                                                       const float* __restrict__ grad_final,
                                                       float* __restrict__ grad_init, float* __restrict__ ws) {
  using L = Ws<D>;
  constexpr int KTW = D / 64, LC = C + 16, LK = D + 16;
  // phase 1: Bq [s][token] and Kc^T [key][token]; phase 2: Qg, W [token][key]
  constexpr int REGION = (C * LC + D * LC) > (2 * C * LK) ? (C * LC + D * LC) : (2 * C * LK);
  __shared__ __align__(16) float sX[REGION];
  __shared__ __align__(16) float sdO[C * 16];
  __shared__ __align__(16) float sdS[D * 16];
  __shared__ __align__(16) float snE[C * 16];
  float* sBq = sX;
  float* sKcT = sX + C * LC;
  float* sQg = sX;
  float* sW = sX + C * LK;
  int n, h, vt;
  if (!slice_of<D>(N, H, n, h, vt)) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
  const int col = 16 * vt + l16;
  const int64_t bos = cu[n], eos = cu[n + 1];
  const int nch = (int)((eos - bos + C - 1) / C);
  const int64_t slot0 = bos / C + n;
  const int64_t sbase = (((int64_t)n * H + h) * D + col) * D;

  f32x4 dS[KTW];
#pragma unroll
  for (int kt = 0; kt < KTW; ++kt) {
    const int key0 = 16 * (w * KTW + kt) + 4 * g;
    dS[kt] = grad_final ? *reinterpret_cast<const f32x4*>(grad_final + sbase + key0) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int c = nch - 1; c >= 0; --c) {
    float* B = ws + ((slot0 + c) * H + h) * L::FLOATS;
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int key0 = 16 * (w * KTW + kt) + 4 * g;
      *reinterpret_cast<f32x4*>(B + L::DS + (int64_t)col * D + key0) = dS[kt];
#pragma unroll
      for (int i = 0; i < 4; ++i) sdS[(key0 + i) * 16 + l16] = dS[kt][i];
    }
    for (int idx = tid; idx < C * C / 4; idx += kThreads) {
      const int s = idx / (C / 4), tq = idx % (C / 4);
      *reinterpret_cast<f32x4*>(sBq + s * LC + 4 * tq) = *reinterpret_cast<const f32x4*>(B + L::BQ + s * C + 4 * tq);
    }
    for (int idx = tid; idx < C * D / 4; idx += kThreads) {
      const int r = idx / (D / 4), cq = idx % (D / 4);
      const f32x4 x = *reinterpret_cast<const f32x4*>(B + L::KC + (int64_t)r * D + 4 * cq);
#pragma unroll
      for (int i = 0; i < 4; ++i) sKcT[(4 * cq + i) * LC + r] = x[i];
    }
    if (tid < C * 4) {
      const int r = tid >> 2, qd = tid & 3;
      *reinterpret_cast<f32x4*>(sdO + r * 16 + 4 * qd) =
          *reinterpret_cast<const f32x4*>(B + L::DOX + (int64_t)r * D + 16 * vt + 4 * qd);
    }
    __syncthreads();
    // dE = Bq^T dO + Kc dS for token tile w
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = 0; s < C; s += 4) acc = mfma4(sBq[(s + g) * LC + 16 * w + l16], sdO[(s + g) * 16 + l16], acc);
#pragma unroll 8
    for (int k0 = 0; k0 < D; k0 += 4) acc = mfma4(sKcT[(k0 + g) * LC + 16 * w + l16], sdS[(k0 + g) * 16 + l16], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g + i;
      B[L::DE + (int64_t)r * D + col] = acc[i];
      snE[r * 16 + l16] = -acc[i];
    }
    __syncthreads();
    for (int idx = tid; idx < C * D / 4; idx += kThreads) {
      const int r = idx / (D / 4), cq = idx % (D / 4);
      *reinterpret_cast<f32x4*>(sQg + r * LK + 4 * cq) = *reinterpret_cast<const f32x4*>(B + L::QG + (int64_t)r * D + 4 * cq);
      *reinterpret_cast<f32x4*>(sW + r * LK + 4 * cq) = *reinterpret_cast<const f32x4*>(B + L::W + (int64_t)r * D + 4 * cq);
    }
    __syncthreads();
    // dS <- Diag(gamma) dS + Qg^T dO - W^T dE
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int key0 = 16 * (w * KTW + kt);
#pragma unroll
      for (int i = 0; i < 4; ++i) dS[kt][i] *= B[L::GAM + key0 + 4 * g + i];
#pragma unroll 4
      for (int t = 0; t < C; t += 4) {
        dS[kt] = mfma4(sQg[(t + g) * LK + key0 + l16], sdO[(t + g) * 16 + l16], dS[kt]);
        dS[kt] = mfma4(sW[(t + g) * LK + key0 + l16], snE[(t + g) * 16 + l16], dS[kt]);
      }
    }
    __syncthreads();
  }
  if (grad_init) {
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int key0 = 16 * (w * KTW + kt) + 4 * g;
      *reinterpret_cast<f32x4*>(grad_init + sbase + key0) = dS[kt];
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 4: per-(chunk, head) gradients.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_grad(const int32_t* __restrict__ cu, int N, int H,
                                                     float* __restrict__ ws, float* __restrict__ gq,
                                                     float* __restrict__ gk, float* __restrict__ gv,
                                                     float* __restrict__ gla, float* __restrict__ gbeta) {
  using L = Ws<D>;
  __shared__ __align__(16) float lds[kGemmLds];
  const int64_t item = blockIdx.x, slot = item / H;
  const int h = (int)(item % H);
  int n, len;
  int64_t t0;
  if (!decode_slot(cu, N, slot, n, t0, len)) return;
  float* B = ws + item * L::FLOATS;
  const float* beta = B + L::BETA;
  double* dG = reinterpret_cast<double*>(B + L::DG);
  auto at = [&](int64_t base, int r, int c) -> float& { return B[base + (int64_t)r * D + c]; };
  // dG accumulates exact fp64 products of fp32 factors
  auto addG = [&](int r, int c, float x, int64_t factor) {
    dG[(int64_t)r * D + c] += (double)x * (double)at(factor, r, c);
  };

  // dQg = dO S0^T: dQ = dQg e^G, dG = dQg o Qg
  wg_gemm<D>(Mat{B + L::DOX, D, 1}, Mat{B + L::S0, D, 1}, D, lds, [&](int r, int c, float x) {
    at(L::DQ, r, c) = x * at(L::EG, r, c);
    dG[(int64_t)r * D + c] = (double)x * (double)at(L::QG, r, c);
  });
  // dKc = E dS_end^T: dK = dKc e^(gC-G), dG -= dKc o Kc
  wg_gemm<D>(Mat{B + L::E, D, 1}, Mat{B + L::DS, D, 1}, D, lds, [&](int r, int c, float x) {
    at(L::DKC, r, c) = x;
    at(L::DK, r, c) = x * at(L::EC, r, c);
    addG(r, c, -x, L::KC);
  });
  // dW = -dE S0^T
  wg_gemm<D>(Mat{B + L::DE, D, 1}, Mat{B + L::S0, D, 1}, D, lds,
             [&](int r, int c, float x) { at(L::DW, r, c) = -x; });
  // dBq = lower(dO E^T), kept as its strict lower part and its diagonal:
  // Bq[r][r] = q_r . k_r carries no decay, so its terms would enter dG twice
  // with opposite signs; they go straight to dq and dk instead
  wg_gemm<C>(Mat{B + L::DOX, D, 1}, Mat{B + L::E, 1, D}, D, lds, [&](int r, int s, float x) {
    B[L::DBQ + r * C + s] = s < r ? x : 0.f;
    if (s == r) B[L::DBQD + r] = x;
  });
  // P = T^T dE: dV = Diag(beta) P
  wg_gemm<D>(Mat{B + L::T, 1, C}, Mat{B + L::DE, D, 1}, C, lds, [&](int r, int c, float x) {
    at(L::P, r, c) = x;
    if (r < len) gv[((t0 + r) * H + h) * D + c] = beta[r] * x;
  });
  // R = T^T dW: dKg = Diag(beta) R: dK += dKg e^G, dG += dKg o Kg
  wg_gemm<D>(Mat{B + L::T, 1, C}, Mat{B + L::DW, D, 1}, C, lds, [&](int r, int c, float x) {
    at(L::R, r, c) = x;
    const float dkg = beta[r] * x;
    at(L::DK, r, c) += dkg * at(L::EG, r, c);
    addG(r, c, dkg, L::KG);
  });
  // dT = dE (Diag(beta) V)^T + dW (Diag(beta) Kg)^T
  wg_gemm<C>(Mat{B + L::DE, D, 1}, Mat{B + L::VX, 1, D}, D, lds,
             [&](int r, int s, float x) { B[L::DT + r * C + s] = beta[s] * x; });
  wg_gemm<C>(Mat{B + L::DW, D, 1}, Mat{B + L::KG, 1, D}, D, lds,
             [&](int r, int s, float x) { B[L::DT + r * C + s] += beta[s] * x; });
  // X = dT T^T; dM = -T^T X: dA = strict_lower(Diag(beta) dM), dMA = strict_lower(dM) o A
  wg_gemm<C>(Mat{B + L::DT, C, 1}, Mat{B + L::T, 1, C}, C, lds,
             [&](int r, int s, float x) { B[L::X + r * C + s] = x; });
  wg_gemm<C>(Mat{B + L::T, 1, C}, Mat{B + L::X, C, 1}, C, lds, [&](int r, int s, float x) {
    const float dm = -x;
    B[L::DA + r * C + s] = s < r ? beta[r] * dm : 0.f;
    B[L::DMA + r * C + s] = s < r ? dm * B[L::A + r * C + s] : 0.f;
  });
  // dKa = dA Kb: dK += dKa e^(G-a), dG += dKa o Ka
  wg_gemm<D>(Mat{B + L::DA, C, 1}, Mat{B + L::KB, D, 1}, C, lds, [&](int r, int c, float x) {
    at(L::DK, r, c) += x * at(L::EGA, r, c);
    addG(r, c, x, L::KA);
  });
  // dKb = dA^T Ka + dBq^T Qa (strict parts): dK += dKb e^(a-G), dG -= dKb o Kb
  wg_gemm<D>(Mat{B + L::DA, 1, C}, Mat{B + L::KA, D, 1}, C, lds, [&](int r, int c, float x) {
    at(L::DK, r, c) += x * at(L::EAG, r, c);
    addG(r, c, -x, L::KB);
  });
  wg_gemm<D>(Mat{B + L::DBQ, 1, C}, Mat{B + L::QA, D, 1}, C, lds, [&](int r, int c, float x) {
    at(L::DK, r, c) += x * at(L::EAG, r, c);
    addG(r, c, -x, L::KB);
  });
  // dQa = dBq Kb (strict part): dQ += dQa e^(G-a), dG += dQa o Qa
  wg_gemm<D>(Mat{B + L::DBQ, C, 1}, Mat{B + L::KB, D, 1}, C, lds, [&](int r, int c, float x) {
    at(L::DQ, r, c) += x * at(L::EGA, r, c);
    addG(r, c, x, L::QA);
  });

  // element-wise assembly: thread c < D owns key channel c
  const int tid = threadIdx.x;
  if (tid < D) {
    const int c = tid;
    double dgam = 0.0;
    for (int j = 0; j < D; ++j)
      dgam += (double)B[L::DS + (int64_t)j * D + c] * (double)B[L::S0 + (int64_t)j * D + c];
    double dgc = dgam * (double)B[L::GAM + c];
    for (int r = 0; r < C; ++r) dgc += (double)at(L::DKC, r, c) * (double)at(L::KC, r, c);
    double suf = 0.0;
    for (int r = C - 1; r >= 0; --r) {
      suf += dG[(int64_t)r * D + c];
      if (r < len) {
        const int64_t o = ((t0 + r) * H + h) * D + c;
        const float dd = B[L::DBQD + r];
        gla[o] = (float)(suf + dgc);
        gq[o] = at(L::DQ, r, c) + dd * at(L::KX, r, c);
        gk[o] = at(L::DK, r, c) + dd * at(L::QX, r, c);
      }
    }
  } else if (tid < D + C) {
    const int r = tid - D;
    if (r < len) {
      float db = 0.f;
      for (int j = 0; j < D; ++j) db += at(L::P, r, j) * at(L::VX, r, j) + at(L::R, r, j) * at(L::KG, r, j);
      for (int s = 0; s < r; ++s) db += B[L::DMA + r * C + s];
      gbeta[(t0 + r) * H + h] = db;
    }
  }
}

template <int D, class In>
static hipError_t launch_t(const BackwardArgs& A, hipStream_t stream) {
  const int64_t slots = prefill_num_slots(A.num_seqs, A.total_tokens);
  const int64_t items = slots * A.num_heads;
  float* ws = (float*)A.workspace;
  if (A.total_tokens > 0) {
    hipLaunchKernelGGL((bwd_prep<D, In>), dim3((unsigned)items), dim3(kThreads), 0, stream, (const In*)A.q,
                       (const In*)A.k, (const In*)A.v, A.log_alpha, (const In*)A.beta, (const In*)A.grad_o,
                       A.cu_seqlens, A.num_seqs, A.num_heads, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t pairs = (int64_t)A.num_seqs * A.num_heads;
  const unsigned blocks = (unsigned)(((pairs + 7) / 8) * 8 * (D / 16));
  if (A.total_tokens > 0) {
    hipLaunchKernelGGL((bwd_fwd<D>), dim3(blocks), dim3(kThreads), 0, stream, A.cu_seqlens, A.num_seqs,
                       A.num_heads, A.init_state, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((bwd_dstate<D>), dim3(blocks), dim3(kThreads), 0, stream, A.cu_seqlens, A.num_seqs,
                     A.num_heads, A.grad_final_state, A.grad_init_state, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || A.total_tokens == 0) return e;
  hipLaunchKernelGGL((bwd_grad<D>), dim3((unsigned)items), dim3(kThreads), 0, stream, A.cu_seqlens, A.num_seqs,
                     A.num_heads, ws, A.grad_q, A.grad_k, A.grad_v, A.grad_log_alpha, A.grad_beta);
  return hipGetLastError();
}

}  // namespace bwd

size_t backward_block_bytes(int d) {
  return (d == 128 ? bwd::Ws<128>::FLOATS : bwd::Ws<64>::FLOATS) * sizeof(float);
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.bf16 ? bwd::launch_t<128, __bf16>(a, stream) : bwd::launch_t<128, float>(a, stream);
  return a.bf16 ? bwd::launch_t<64, __bf16>(a, stream) : bwd::launch_t<64, float>(a, stream);
}

}  // namespace kda
