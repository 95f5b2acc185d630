// kda_prefill_bf16.hip -- chunk-parallel KDA prefill for bf16 inputs.
//
// Same chunk equations as kda_prefill.hip (derived from the recurrence of
// the page "Kimi Delta Attention", §03, over chunks of C = 64 tokens, §06),
// with the read-out regrouped so that the sequential pass needs no
// intra-chunk product:
//
//   O = Qg S0 + Bqk E = Qg S0 + Bqk (U - W S0) = Q' S0 + Bqk U,
//   Q' = Qg - Bqk W          (computed per chunk, in parallel)
//
// Kernel 1 (prep) is persistent: each workgroup walks (chunk, head) items
// and loads the raw inputs of its next item into registers while it
// computes the current one.  Per item it produces, as MFMA fragments:
// W, Q' and Kc^T (fp16), U and Bqk U (fp32 accumulator tiles) and e^G[C-1].
//
// Precision (fp32 accumulation throughout).  Inside the prep, an operand
// whose bf16 rounding would show in the outputs is split into hi + lo bf16
// parts and multiplied as hi*hi + hi*lo + lo*hi: Q and K scaled by the decay
// in Q K^T (the intra-chunk matrix Bqk), Bqk itself and U in Bqk U.  The
// K K^T operands, T and Kg stay single bf16.  The decay-scaled operands
// there span up to e^(+-80) (the anchor sits mid-chunk), which only bf16
// covers.  The operands of the sequential pass -- W, Q', Kc, S and E -- are
// all of moderate size and go through single fp16 (11-bit significand).
//
// Kernel 2 (state pass) is one workgroup per (sequence, head, 16 value
// columns): S's columns never mix in the recurrence.  Per chunk:
//   E = U - W S;  O = Q' S + Bqk U;  S <- Diag(e^G[C-1]) S + Kc^T E.
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_prefill_common.h"

namespace kda {
namespace bf {

using In = __bf16;
using Frag = bf16x8;
using Half = bf16x4;
using HFrag = f16x8;    // fp16 operands of the sequential pass
using HHalf = f16x4;
using SplitB = Split<PathBF16>;
constexpr int C = kChunk;
constexpr size_t FB = 64 * sizeof(Frag);   // bytes per fragment
constexpr int kPrepThreads = 512;

// Per (chunk slot, head) record.
template <int D>
struct Rec {
  static constexpr int KB = D / 32, NT = D / 16;
  static constexpr size_t W = 0;                             // [4 token tiles][KB]          W
  static constexpr size_t QP = W + 4 * KB * FB;              // [4 token tiles][KB]          Q'
  static constexpr size_t KC = QP + 4 * KB * FB;             // [NT key tiles][2]            Kc^T
  static constexpr size_t U = KC + NT * 2 * FB;              // [NT value tiles][4 token tiles][64] f32x4
  static constexpr size_t BU = U + (size_t)NT * 4 * 64 * 16; // same layout, Bqk U
  static constexpr size_t G = BU + (size_t)NT * 4 * 64 * 16; // [D] fp32 e^G[C-1]
  static constexpr size_t BYTES = G + (size_t)D * 4;
};

// Raw inputs of one item held in registers, token-major, as 16-byte vectors
// (K, Q, V rows in bf16, log_alpha rows in fp32), and beta for one token.
template <int D>
struct Prefetch {
  static constexpr int VR = D / 8;                      // bf16 vectors per row
  static constexpr int NVT = C * VR / kPrepThreads;     // bf16 vectors per thread and tensor
  static constexpr int VRA = D / 4;                     // fp32 vectors per row
  static constexpr int NVA = C * VRA / kPrepThreads;    // fp32 vectors per thread
  static constexpr int SEGS = kPrepThreads / D;         // token runs per channel (cumulative sum)
  static constexpr int SL = C / SEGS;                   // tokens per run
  uint4 k[NVT], q[NVT], v[NVT];
  f32x4 la[NVA];
  float beta;
};

template <int D>
__device__ __forceinline__ void prefetch(Prefetch<D>& f, const In* __restrict__ q, const In* __restrict__ k,
                                         const In* __restrict__ v, const float* __restrict__ la,
                                         const In* __restrict__ beta, int H, int h, int64_t t0, int len,
                                         int tid) {
  using F = Prefetch<D>;
  const int64_t base = (t0 * H + h) * D;   // first element of the item's rows
  const int pitch = H * D;                 // elements between consecutive tokens
#pragma unroll
  for (int i = 0; i < F::NVT; ++i) {
    const int idx = tid + i * kPrepThreads;
    const int r = idx / F::VR, cv = idx % F::VR;
    f.k[i] = f.q[i] = f.v[i] = uint4{0, 0, 0, 0};
    if (r < len) {
      const int off = r * pitch + cv * 8;
      f.k[i] = *reinterpret_cast<const uint4*>(k + base + off);
      f.q[i] = *reinterpret_cast<const uint4*>(q + base + off);
      f.v[i] = *reinterpret_cast<const uint4*>(v + base + off);
    }
  }
#pragma unroll
  for (int i = 0; i < F::NVA; ++i) {
    const int idx = tid + i * kPrepThreads;
    const int r = idx / F::VRA, cv = idx % F::VRA;
    f.la[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r < len) f.la[i] = *reinterpret_cast<const f32x4*>(la + base + r * pitch + cv * 4);
  }
  f.beta = (tid < len) ? (float)beta[(t0 + tid) * H + h] : 0.f;
}

// next (chunk slot, head) item of this workgroup that holds tokens
__device__ __forceinline__ int64_t next_item(const int32_t* __restrict__ cu, int N, int H, int64_t it,
                                             int64_t n_items, int& n, int64_t& t0, int& len) {
  for (; it < n_items; it += gridDim.x)
    if (decode_slot(cu, N, it / H, n, t0, len)) return it;
  return n_items;
}

// ---------------------------------------------------------------------------
// Kernel 1: per-chunk factors (persistent).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ log_alpha, const In* __restrict__ beta, const int32_t* __restrict__ cu,
    int N, int H, int64_t n_items, unsigned char* __restrict__ ws) {
  using R = Rec<D>;
  using F = Prefetch<D>;
  constexpr int KB = D / 32, NT = D / 16;
  constexpr int NW = kPrepThreads / 64;
  constexpr int PI = D + 8;   // bf16 row pitch (+16 bytes)
  constexpr int PX = D + 4;   // fp32 row pitch (+16 bytes)
  constexpr int PL = C + 4;
  constexpr int SEGS = F::SEGS, SL = F::SL;
  constexpr size_t KBYTES = (size_t)C * PI * 2 > 16 * FB ? (size_t)C * PI * 2 : 16 * FB;
  constexpr size_t LBYTES = (size_t)C * PL * 4;   // one 64 x 64 fp32 matrix
  constexpr size_t BIGBYTES = 2 * LBYTES + 8 * FB > 40 * FB ? 2 * LBYTES + 8 * FB : 40 * FB;

  __shared__ __align__(16) unsigned char sKraw[KBYTES];   // K rows; then Bqk fragments
  __shared__ __align__(16) In sQ[C][PI];
  __shared__ __align__(16) float sX[C][PX];               // X = e^(G - G[31])
  // key-block staging (two buffers of 20 fragments) during P3; afterwards
  // L = Diag(beta) A (strictly lower), T and the T' fragments
  __shared__ __align__(16) unsigned char sBig[BIGBYTES];
  __shared__ __align__(16) Frag sKg[NT][2][64];           // Kg^T fragments (row key, k token)
  __shared__ __align__(16) In sV[C][PI];                  // V rows
  __shared__ __align__(16) float sLdT[4][16][20];         // diagonal 16-blocks of L, transposed
  __shared__ float sEgm[D], sEcm[D], sGm[D], sGc[D], sBeta[C];
  __shared__ float sSeg[SEGS][D];
  __shared__ __align__(16) float sScr[4][16][20];
  auto sK = reinterpret_cast<In (*)[PI]>(sKraw);
  auto sBq = reinterpret_cast<Frag (*)[4][2][64]>(sKraw);       // [hi,lo][row tile][token block][lane]
  auto sStage = reinterpret_cast<Frag (*)[20][64]>(sBig);       // [buffer][fragment][lane]
  auto sL = reinterpret_cast<float (*)[PL]>(sBig);
  auto sT = reinterpret_cast<float (*)[PL]>(sBig + LBYTES);
  auto sTf = reinterpret_cast<Frag (*)[2][64]>(sBig + 2 * LBYTES);   // T' [row tile][token block]

  int n, len;
  int64_t t0;
  int64_t item = next_item(cu, N, H, blockIdx.x, n_items, n, t0, len);
  F pf;
  if (item < n_items) prefetch<D>(pf, q, k, v, log_alpha, beta, H, (int)(item % H), t0, len, threadIdx.x);

  while (item < n_items) {
    // The thread index is re-read through an opaque move each item so that
    // the many lane-dependent LDS addresses are formed inside the loop
    // instead of being hoisted out of it and spilled.
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, l16 = l & 15;
    const int ch = tid % D, sg = tid / D;
    const int64_t slot = item / H;
    const int h = (int)(item % H);
    unsigned char* rec = ws + ((size_t)slot * H + h) * R::BYTES;

    // ---- P1: prefetched rows to LDS (log_alpha into the X buffer, V into
    //      its fragments); running sums of log_alpha -------------------------
#pragma unroll
    for (int i = 0; i < F::NVT; ++i) {
      const int idx = tid + i * kPrepThreads;
      const int r = idx / F::VR, cv = idx % F::VR;
      *reinterpret_cast<uint4*>(&sK[r][cv * 8]) = pf.k[i];
      *reinterpret_cast<uint4*>(&sQ[r][cv * 8]) = pf.q[i];
      *reinterpret_cast<uint4*>(&sV[r][cv * 8]) = pf.v[i];
    }
#pragma unroll
    for (int i = 0; i < F::NVA; ++i) {
      const int idx = tid + i * kPrepThreads;
      const int r = idx / F::VRA, cv = idx % F::VRA;
      *reinterpret_cast<f32x4*>(&sX[r][cv * 4]) = pf.la[i];
    }
    if (tid < C) sBeta[tid] = pf.beta;
    int n2, len2;
    int64_t t02;
    const int64_t item2 = next_item(cu, N, H, item + gridDim.x, n_items, n2, t02, len2);
    __syncthreads();

    // ---- P2: cumulative log decay; X; Kg^T and Kc^T fragments --------------
    {
      float gl[SL];
      {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < SL; ++r) {
          run += sX[sg * SL + r][ch];
          gl[r] = run;
        }
        sSeg[sg][ch] = run;
      }
      __syncthreads();
      float off = 0.f;
      for (int s2 = 0; s2 < sg; ++s2) off += sSeg[s2][ch];
#pragma unroll
      for (int r = 0; r < SL; ++r) gl[r] += off;
      if (sg == 31 / SL) sGm[ch] = gl[31 % SL];
      if (sg == SEGS - 1) sGc[ch] = gl[SL - 1];
      __syncthreads();
      const float gm = sGm[ch], gc = sGc[ch];
      const float egm = __expf(gm), ecm = __expf(gc - gm);
      if (sg == 0) {
        sEgm[ch] = egm;
        sEcm[ch] = ecm;
        reinterpret_cast<float*>(rec + R::G)[ch] = __expf(gc);
      }
      // this channel is key ch: key tile ch/16, fragment row ch%16.  Four
      // consecutive tokens j0..j0+3 of a 32-token block sit at fragment
      // positions 4*hh .. 4*hh+3 of lane row + 16*gp.
      const int tile = ch >> 4, rowl = ch & 15;
#pragma unroll
      for (int r0 = 0; r0 < SL; r0 += 4) {
        const int j0 = sg * SL + r0;
        const int p = j0 >> 5, jj = j0 & 31, gp = (jj & 15) >> 2, hh = jj >> 4;
        const int lane = rowl + 16 * gp;
        Half kg4;
        HHalf kc4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + e;
          const float x = __expf(gl[r0 + e] - gm);
          sX[j][ch] = x;
          const float kx = (float)sK[j][ch];
          kg4[e] = (In)(kx * x * egm);
          kc4[e] = (_Float16)(kx * __builtin_amdgcn_rcpf(x) * ecm);
        }
        *reinterpret_cast<Half*>(reinterpret_cast<In*>(&sKg[tile][p][lane]) + 4 * hh) = kg4;
        const int koff = ((tile * 2 + p) * 64 + lane) * 16 + 8 * hh;
        *reinterpret_cast<HHalf*>(rec + R::KC + koff) = kc4;
      }
    }
    __syncthreads();

    // ---- P3: A = Ka Kbar^T and Bqk^T = Kbar Qa^T, one key block at a time --
    {
      f32x4 accA[2], accB[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        accA[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        accB[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // staging slots: 0..3 Ka, 4..7 Kbar hi, 8..11 Kbar lo, 12..15 Qa hi,
      // 16..19 Qa lo; key block p+1 is built while block p is multiplied
      // wave w builds half hh = w / 4 (keys 16 hh .. 16 hh + 15 of the block)
      // of Ka, Kbar and Qa for row tile w % 4, reading K, Q and X once
      auto build = [&](int p, int buf) {
        const int rt = w & 3, hh = w >> 2;
        const int row = 16 * rt + l16, key = 32 * p + 16 * hh + 4 * g;
        const f32x4 kv = lds4(&sK[row][key]), qv = lds4(&sQ[row][key]);
        const f32x4 x = *reinterpret_cast<const f32x4*>(&sX[row][key]);
        Half ka, kbh, kbl, qah, qal;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = kv[e] * x[e];
          const float kb = kv[e] * __builtin_amdgcn_rcpf(x[e]);
          const float qa = qv[e] * x[e];
          ka[e] = (In)a;
          kbh[e] = (In)kb;
          kbl[e] = (In)(kb - (float)kbh[e]);
          qah[e] = (In)qa;
          qal[e] = (In)(qa - (float)qah[e]);
        }
        auto put = [&](int slot, const Half& hv) {
          *reinterpret_cast<Half*>(reinterpret_cast<In*>(&sStage[buf][slot][l]) + 4 * hh) = hv;
        };
        put(rt, ka);
        put(4 + rt, kbh);
        put(8 + rt, kbl);
        put(12 + rt, qah);
        put(16 + rt, qal);
      };
      build(0, 0);
      __syncthreads();
      for (int p = 0; p < KB; ++p) {
        if (p + 1 < KB) build(p + 1, (p + 1) & 1);
        const int buf = p & 1;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int pi = w + NW * i;
          if (pi < 10) {
            const int rt = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
            const int jt = pi - (rt * (rt + 1)) / 2;
            const Frag kbh = sStage[buf][4 + jt][l], kbl = sStage[buf][8 + jt][l];
            const Frag qah = sStage[buf][12 + rt][l], qal = sStage[buf][16 + rt][l];
            mma(accA[i], sStage[buf][rt][l], kbh);   // A[r][j]
            mma(accB[i], kbh, qah);                  // Bqk^T[j][r]
            mma(accB[i], kbh, qal);
            mma(accB[i], kbl, qah);
          }
        }
        __syncthreads();
      }
      // A -> Diag(beta) A (strictly lower) in sL; Bqk -> split fragments
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int pi = w + NW * i;
        if (pi < 10) {
          const int rt = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
          const int jt = pi - (rt * (rt + 1)) / 2;
          Half hb, lb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * rt + 4 * g + e, j = 16 * jt + l16;
            const float lv = (j < r) ? sBeta[r] * accA[i][e] : 0.f;
            sL[r][j] = lv;
            if (jt == rt) sLdT[rt][l16][4 * g + e] = lv;   // column j of the block as a row
            // Bqk^T tile: lane holds Bqk[16 rt + l16][16 jt + 4 g + e]
            const int rr = 16 * rt + l16, jj = 16 * jt + 4 * g + e;
            const float x = jj <= rr ? accB[i][e] : 0.f;
            hb[e] = (In)x;
            lb[e] = (In)(x - (float)hb[e]);
          }
          *reinterpret_cast<Half*>(reinterpret_cast<In*>(&sBq[0][rt][jt >> 1][l]) + 4 * (jt & 1)) = hb;
          *reinterpret_cast<Half*>(reinterpret_cast<In*>(&sBq[1][rt][jt >> 1][l]) + 4 * (jt & 1)) = lb;
          if (jt == rt && (rt & 1) == 0) {   // the half above the diagonal block
            const Half z = {(In)0.f, (In)0.f, (In)0.f, (In)0.f};
            *reinterpret_cast<Half*>(reinterpret_cast<In*>(&sBq[0][rt][jt >> 1][l]) + 4) = z;
            *reinterpret_cast<Half*>(reinterpret_cast<In*>(&sBq[1][rt][jt >> 1][l]) + 4) = z;
          }
        }
      }
    }
    __syncthreads();

    // ---- P4: T = (I + L)^-1 ---------------------------------------------------
    // 16 x 16 diagonal blocks by column-oriented forward substitution, then
    // block doubling  [[X, 0], [Y, Z]]^-1 = [[X^-1, 0], [-Z^-1 Y X^-1, Z^-1]]
    // for the 16-blocks (1,0), (3,2) and then the 32-block (1,0).  The block
    // products run on v_mfma_f32_16x16x4_f32 with the reduction index of
    // instruction s taken as 4 g + s, so that a row of the left factor is
    // one 16-byte LDS read and the right factor is an accumulator tile.
    {
      // the next item's inputs are in flight from here on (most waves are
      // idle in this phase)
      if (item2 < n_items) prefetch<D>(pf, q, k, v, log_alpha, beta, H, (int)(item2 % H), t02, len2, tid);
      for (int idx = tid; idx < C * PL; idx += kPrepThreads) (&sT[0][0])[idx] = 0.f;
      const int bk = l >> 4, cc = l & 15;   // wave 0: lane = (block, column)
      float x[16];
      if (w == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == cc) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 15; ++j) {
          f32x4 colj[4];   // column j of the block: L[r][j], r = 0..15
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) colj[qd] = *reinterpret_cast<const f32x4*>(&sLdT[bk][j][4 * qd]);
#pragma unroll
          for (int r = j + 1; r < 16; ++r) x[r] -= colj[r >> 2][r & 3] * x[j];
        }
      }
      __syncthreads();   // sT cleared
      if (w == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[16 * bk + r][16 * bk + cc] = x[r];
      }
      __syncthreads();
      const int c = l16;
      // accumulator tile (rows 4g+e, column c) of block (R, K) of sT
      auto ctile = [&](int R, int K) {
        f32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = sT[16 * R + 4 * g + e][16 * K + c];
        return t;
      };
      // acc += M[16 R + row][16 K + k] * B[k][col] for the 16-block (R, K) of an LDS matrix
      auto mma_rows = [&](f32x4& acc, const float (*M)[PL], int R, int K, const f32x4& b) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&M[16 * R + l16][16 * K + 4 * g]);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s4], b[s4], acc, 0, 0, 0);
      };
      if (w < 2) {   // T(bb, a) = -T(bb, bb) L(bb, a) T(a, a), bb = a + 1
        const int a = 2 * w, bb = a + 1;
        f32x4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
        mma_rows(y, sL, bb, a, ctile(a, a));
        mma_rows(z, sT, bb, bb, y);
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[16 * bb + 4 * g + e][16 * a + c] = -z[e];
      }
      __syncthreads();
      // Y = L[32:64, 0:32] T[0:32, 0:32]; T[32:64, 0:32] = -T[32:64, 32:64] Y;
      // wave w < 4 owns 16-tile (bi, bj)
      if (w < 4) {
        const int bi = w >> 1, bj = w & 1;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        for (int kb = bj; kb < 2; ++kb) mma_rows(y, sL, 2 + bi, kb, ctile(kb, bj));
#pragma unroll
        for (int e = 0; e < 4; ++e) sScr[w][4 * g + e][c] = y[e];
      }
      __syncthreads();
      if (w < 4) {
        const int bi = w >> 1, bj = w & 1;
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb <= bi; ++kb) {
          f32x4 yt;
#pragma unroll
          for (int e = 0; e < 4; ++e) yt[e] = sScr[2 * kb + bj][4 * g + e][c];
          mma_rows(z, sT, 2 + bi, 2 + kb, yt);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[32 + 16 * bi + 4 * g + e][16 * bj + c] = -z[e];
      }
      __syncthreads();
      // T' = T Diag(beta) fragments (row tile rt, token block p), one per wave
      {
        const int rt = w >> 1, p = w & 1;
        float vals[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int j = 32 * p + kpos(g, m);
          vals[m] = sT[16 * rt + l16][j] * sBeta[j];
        }
        sTf[rt][p][l] = make_frag<PathBF16>(vals);
      }
      __syncthreads();
    }

    // ---- P5: W, Q' = Qg - Bqk W, U = T' V, Bqk U -------------------------------
    for (int task = w; task < 2 * NT; task += NW) {
      if (task < NT) {
        const int it = task;   // key tile
        f32x4 wc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          f32x4 wt = {0.f, 0.f, 0.f, 0.f};
          wc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (p > (rt >> 1)) break;   // T'[r][j] = 0 for j > r
            const Frag tf = sTf[rt][p][l], kg = sKg[it][p][l];
            mma(wc[rt], tf, kg);   // W[r][i]
            mma(wt, kg, tf);       // W^T[i][r]
          }
          HHalf hw;
#pragma unroll
          for (int e = 0; e < 4; ++e) hw[e] = (_Float16)wt[e];
          *reinterpret_cast<HHalf*>(rec + R::W + ((rt * KB + (it >> 1)) * 64 + l) * 16 + 8 * (it & 1)) = hw;
        }
        // -W^T as the A operand over token block p (from the W tiles 2p, 2p+1)
        Frag wn[2];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            wn[p][e] = (In)(-wc[2 * p][e]);
            wn[p][4 + e] = (In)(-wc[2 * p + 1][e]);
          }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          // Q'^T tile (key tile it, token tile rt), started from Qg^T
          const int r = 16 * rt + l16, k0 = 16 * it + 4 * g;
          const f32x4 q4 = lds4(&sQ[r][k0]);
          const f32x4 x4 = *reinterpret_cast<const f32x4*>(&sX[r][k0]);
          f32x4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = q4[e] * x4[e] * sEgm[k0 + e];
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (p > (rt >> 1)) break;   // Bqk[r][j] = 0 for j > r
            mma(acc, wn[p], sBq[0][rt][p][l]);
            mma(acc, wn[p], sBq[1][rt][p][l]);
          }
          HHalf hq;
#pragma unroll
          for (int e = 0; e < 4; ++e) hq[e] = (_Float16)acc[e];
          const int qo = ((rt * KB + (it >> 1)) * 64 + l) * 16 + 8 * (it & 1);
          *reinterpret_cast<HHalf*>(rec + R::QP + qo) = hq;
        }
      } else {
        const int ct = task - NT;   // value tile
        Frag vf[2];                 // V fragments (col value, k token)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int m = 0; m < 8; ++m) vf[p][m] = sV[32 * p + kpos(g, m)][16 * ct + l16];
        f32x4 uc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          uc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (p > (rt >> 1)) break;
            mma(uc[rt], sTf[rt][p][l], vf[p]);
          }
          *reinterpret_cast<f32x4*>(rec + R::U + ((ct * 4 + rt) * 64 + l) * 16) = uc[rt];
        }
        // U as the B operand over token block p, split
        SplitB ub[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float vals[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vals[e] = uc[2 * p][e];
            vals[4 + e] = uc[2 * p + 1][e];
          }
          ub[p] = make_split<PathBF16>(vals);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          f32x4 bu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (p > (rt >> 1)) break;
            const Frag bh = sBq[0][rt][p][l], bl = sBq[1][rt][p][l];
            mma(bu, bh, ub[p].hi);
            mma(bu, bh, ub[p].lo);
            mma(bu, bl, ub[p].hi);
          }
          *reinterpret_cast<f32x4*>(rec + R::BU + ((ct * 4 + rt) * 64 + l) * 16) = bu;
        }
      }
    }
    __syncthreads();   // LDS is reused by the next item

    item = item2;
    n = n2;
    t0 = t02;
    len = len2;
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: sequential pass over the chunks of one (sequence, head) for a
// 16-column slice of S.  Wave w owns key rows [D/4 w, D/4 (w+1)) of the
// slice as accumulators and token tile w of every chunk; the operands of
// the next two chunks are in flight while the current one is computed.
// ---------------------------------------------------------------------------
template <int D>
struct Ops {
  static constexpr int KB = D / 32, KTW = D / 64;
  HFrag w[KB];           // W, token tile of this wave
  HFrag qp[KB];          // Q', token tile of this wave
  HFrag kc[KTW][2];      // Kc^T for this wave's key tiles
  f32x4 u, bu;           // U and Bqk U, token tile of this wave, this slice
  f32x4 gam[KTW];        // e^G[C-1] for this lane's key rows
};

// The operand loads of one chunk, in three parts that the step spreads over
// its phases so that the vector memory path works while the MFMAs do.
template <int D>
__device__ __forceinline__ void load_ops_part(Ops<D>& o, const unsigned char* __restrict__ rec, int part, int w,
                                              int l, int g, int vt) {
  using R = Rec<D>;
  using O = Ops<D>;
  if (part == 0) {
#pragma unroll
    for (int p = 0; p < O::KB; ++p)
      o.w[p] = *reinterpret_cast<const HFrag*>(rec + R::W + ((w * O::KB + p) * 64 + l) * 16);
    o.u = *reinterpret_cast<const f32x4*>(rec + R::U + ((vt * 4 + w) * 64 + l) * 16);
    o.bu = *reinterpret_cast<const f32x4*>(rec + R::BU + ((vt * 4 + w) * 64 + l) * 16);
  } else if (part == 1) {
#pragma unroll
    for (int p = 0; p < O::KB; ++p)
      o.qp[p] = *reinterpret_cast<const HFrag*>(rec + R::QP + ((w * O::KB + p) * 64 + l) * 16);
  } else {
#pragma unroll
    for (int kt = 0; kt < O::KTW; ++kt)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int kti = w * O::KTW + kt;
        o.kc[kt][p] = *reinterpret_cast<const HFrag*>(rec + R::KC + ((kti * 2 + p) * 64 + l) * 16);
      }
#pragma unroll
    for (int kt = 0; kt < O::KTW; ++kt)
      o.gam[kt] = *reinterpret_cast<const f32x4*>(rec + R::G + (16 * (w * O::KTW + kt) + 4 * g) * 4);
  }
}

template <int D>
__device__ __forceinline__ void load_ops(Ops<D>& o, const unsigned char* __restrict__ rec, int w, int l, int g,
                                         int vt) {
#pragma unroll
  for (int part = 0; part < 3; ++part) load_ops_part<D>(o, rec, part, w, l, g, vt);
}

template <int D>
__global__ __launch_bounds__(kThreads) void state_kernel(const int32_t* __restrict__ cu, int N, int H,
                                                         const float* init, float* fin, In* __restrict__ o,
                                                         const unsigned char* __restrict__ ws) {
  using R = Rec<D>;
  constexpr int NV = D / 16, KB = D / 32, KTW = D / 64;

  // XCD-aware order: the NV slices of one (sequence, head) share an XCD (and
  // its L2) because workgroups are dealt to the 8 XCDs round-robin.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, rest = bid >> 3;
  const int vt = rest % NV;
  const int pair = (rest / NV) * 8 + xcd;
  if (pair >= N * H) return;
  const int n = pair / H, h = pair % H;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
  const int col = 16 * vt + l16;
  const int64_t bos = cu[n], eos = cu[n + 1];
  const int nch = (int)((eos - bos + kChunk - 1) / kChunk);
  const int64_t slot0 = bos / kChunk + n;

  __shared__ HFrag sS[KB][64];   // S as the B operand
  __shared__ HFrag sE[2][64];    // E as the B operand

  const int64_t sbase = ((int64_t)n * H + h) * D;
  f32x4 S[KTW];
#pragma unroll
  for (int kt = 0; kt < KTW; ++kt) {
    const int kti = w * KTW + kt;
    S[kt] = init ? *reinterpret_cast<const f32x4*>(init + (sbase + col) * D + 16 * kti + 4 * g)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto rec_of = [&](int c) { return ws + ((size_t)(slot0 + min(c, nch - 1)) * H + h) * R::BYTES; };

  // one chunk step with operands `ops`; meanwhile the operands of a later
  // chunk (record `nrec`) are loaded into `nxt`, one part per phase
  auto step = [&](const Ops<D>& ops, int c, Ops<D>& nxt, const unsigned char* nrec) {
    load_ops_part<D>(nxt, nrec, 0, w, l, g, vt);
    const int64_t t0 = bos + (int64_t)c * kChunk;
    const int len = (int)min<int64_t>(kChunk, eos - t0);
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int kti = w * KTW + kt;
      HHalf hs;
#pragma unroll
      for (int e = 0; e < 4; ++e) hs[e] = (_Float16)S[kt][e];
      *reinterpret_cast<HHalf*>(reinterpret_cast<_Float16*>(&sS[kti >> 1][l]) + 4 * (kti & 1)) = hs;
    }
    __syncthreads();
    load_ops_part<D>(nxt, nrec, 1, w, l, g, vt);
    // token tile w: W S and Q' S
    f32x4 wsum = {0.f, 0.f, 0.f, 0.f}, qsum = ops.bu;
#pragma unroll
    for (int p = 0; p < KB; ++p) {
      const HFrag sf = sS[p][l];
      mma(wsum, ops.w[p], sf);
      mma(qsum, ops.qp[p], sf);
    }
    // E = U - W S, published as the B operand over tokens
    HHalf eh;
#pragma unroll
    for (int e = 0; e < 4; ++e) eh[e] = (_Float16)(ops.u[e] - wsum[e]);
    *reinterpret_cast<HHalf*>(reinterpret_cast<_Float16*>(&sE[w >> 1][l]) + 4 * (w & 1)) = eh;
    // O = Q' S + Bqk U for token tile w
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * w + 4 * g + e;
      if (r < len) o[((t0 + r) * H + h) * D + col] = (In)qsum[e];
    }
    __syncthreads();
    load_ops_part<D>(nxt, nrec, 2, w, l, g, vt);
    // S <- Diag(e^G[C-1]) S + Kc^T E
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      S[kt] *= ops.gam[kt];
#pragma unroll
      for (int p = 0; p < 2; ++p) mma(S[kt], ops.kc[kt][p], sE[p][l]);
    }
  };

  // three operand buffers in rotation: while chunk c is computed, chunk
  // c+1's operands are in flight and chunk c+2's are being loaded (past the
  // last chunk the last record is read again, so every step issues the same
  // loads and the compiler's waits stay exact)
  Ops<D> bufA, bufB, bufC;
  if (nch > 0) {
    load_ops<D>(bufA, rec_of(0), w, l, g, vt);
    load_ops<D>(bufB, rec_of(1), w, l, g, vt);
  }
  for (int c = 0; c < nch; c += 3) {
    step(bufA, c, bufC, rec_of(c + 2));
    if (c + 1 >= nch) break;
    step(bufB, c + 1, bufA, rec_of(c + 3));
    if (c + 2 >= nch) break;
    step(bufC, c + 2, bufB, rec_of(c + 4));
  }

  if (fin) {
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int kti = w * KTW + kt;
      *reinterpret_cast<f32x4*>(fin + (sbase + col) * D + 16 * kti + 4 * g) = S[kt];
    }
  }
}

template <int D>
static hipError_t launch_t(const PrefillArgs& A, hipStream_t stream) {
  const int64_t slots = prefill_num_slots(A.num_seqs, A.total_tokens);
  const int64_t items = slots * A.num_heads;
  if (A.total_tokens > 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    const unsigned grid = (unsigned)(items < cus ? items : cus);
    hipLaunchKernelGGL((prep_kernel<D>), dim3(grid), dim3(kPrepThreads), 0, stream, (const In*)A.q,
                       (const In*)A.k, (const In*)A.v, A.log_alpha, (const In*)A.beta, A.cu_seqlens,
                       A.num_seqs, A.num_heads, items, (unsigned char*)A.workspace);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t pairs = (int64_t)A.num_seqs * A.num_heads;
  const int64_t groups = (pairs + 7) / 8;
  const unsigned blocks = (unsigned)(groups * 8 * (D / 16));
  hipLaunchKernelGGL((state_kernel<D>), dim3(blocks), dim3(kThreads), 0, stream, A.cu_seqlens, A.num_seqs,
                     A.num_heads, A.init_state, A.final_state, (In*)A.o, (const unsigned char*)A.workspace);
  return hipGetLastError();
}

}  // namespace bf

size_t prefill_record_bytes_bf16(int d) { return d == 128 ? bf::Rec<128>::BYTES : bf::Rec<64>::BYTES; }

hipError_t launch_prefill_bf16(const PrefillArgs& A, hipStream_t stream) {
  if (A.num_seqs == 0) return hipSuccess;
  return A.d == 128 ? bf::launch_t<128>(A, stream) : bf::launch_t<64>(A, stream);
}

}  // namespace kda
