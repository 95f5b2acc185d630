// kda_prefill_bf16.hip -- chunk-parallel KDA prefill for bf16 inputs.
//
// Same chunk equations as kda_prefill.hip (derived from the recurrence of
// the page "Kimi Delta Attention", §03, over chunks of C = 64 tokens, §06),
// with the read-out in one of two groupings:
//
//   O = Qg S0 + Bqk E = Qg S0 + Bqk (U - W S0) = Q' S0 + Bqk U,
//   Q' = Qg - Bqk W          (computed per chunk, in parallel)
//
// The second leaves the sequential pass no intra-chunk product; the first
// leaves the per-chunk work less to do (the pass forms Bqk E from the E it
// already holds), and is used where that work is the longer leg.
//
// The prep runs one workgroup of four waves per (chunk, head) item, two
// workgroups per CU, each wave holding 16 tokens of the chunk in registers.
// Per item it produces, as MFMA fragments: W, Kc^T and e^G[C-1]; U (fp16
// accumulator tiles); and either Q' and (Bqk U)^T or Qg and Bqk.
//
// Precision (fp32 accumulation throughout).  Inside the prep, an operand
// whose bf16 rounding would show in the outputs is split into hi + lo bf16
// parts and multiplied as hi*hi + hi*lo + lo*hi: Q and K scaled by the decay
// in Q K^T (the intra-chunk matrix Bqk), Bqk itself and U in Bqk U.  The
// K K^T operands, T and Kg stay single bf16.  The decay-scaled operands
// there span up to e^(+-80) (the anchor sits mid-chunk), which only bf16
// covers.  The operands of the sequential pass -- W, Q' or Qg, Kc, U,
// Bqk U or Bqk, S and E -- are all of moderate size and go through single
// fp16 (11-bit significand).
//
// The state pass is one task per (sequence, head, slice of value columns):
// S's columns never mix in the recurrence.  Per chunk:
//   E = U - W S;  O = Q' S + Bqk U (or Qg S + Bqk E);  S <- Diag(e^G[C-1]) S + Kc^T E.
#include <algorithm>
#include <cstddef>

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
constexpr int kPrepThreads = 256;

// ---------------------------------------------------------------------------
// Record access.  A record is written by one workgroup and read by others
// that may sit on another XCD, whose L2 is a different cache.  Every record
// store and load therefore carries the SC1 cache-policy bit (device-scope
// coherence, the policy of relaxed agent-scope atomics on gfx950): stores
// reach the device coherence point before they are acknowledged and loads do
// not return a stale copy from the local L1 or a non-coherent L2 line.  A
// flag stored after the stores' acknowledgement then publishes the record
// without a device-wide cache flush (an agent-scope fence writes back and
// invalidates the whole L2, which costs more than the pass itself).
// ---------------------------------------------------------------------------
constexpr int kCoherent = 16;   // SC1
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc rec_rsrc(const unsigned char* rec, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(rec), (short)0, (int)bytes, 0x00020000);
}
template <class T>
__device__ __forceinline__ T ld_rec(Rsrc rs, size_t off) {
  static_assert(sizeof(T) == 16 || sizeof(T) == 8, "record loads are 8 or 16 bytes");
  if constexpr (sizeof(T) == 16) return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, kCoherent));
  else return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, kCoherent));
}
template <class T>
__device__ __forceinline__ void st_rec(Rsrc rs, size_t off, const T& x) {
  static_assert(sizeof(T) == 16 || sizeof(T) == 8 || sizeof(T) == 4, "record stores are 4, 8 or 16 bytes");
  if constexpr (sizeof(T) == 16) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs, (int)off, 0, kCoherent);
  else if constexpr (sizeof(T) == 8) __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), rs, (int)off, 0, kCoherent);
  else __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), rs, (int)off, 0, kCoherent);
}

// Per (chunk slot, head) record.
template <int D>
struct Rec {
  static constexpr int KB = D / 32, NT = D / 16;
  static constexpr size_t W = 0;                             // [4 token tiles][KB]          W
  static constexpr size_t QP = W + 4 * KB * FB;              // [4 token tiles][KB]          Q' (or Qg)
  static constexpr size_t KC = QP + 4 * KB * FB;             // [NT key tiles][2]            Kc^T
  static constexpr size_t U = KC + NT * 2 * FB;              // [NT value tiles][4 token tiles][64] f16x4
  static constexpr size_t BU = U + (size_t)NT * 4 * 64 * 8;  // same tiles of (Bqk U)^T: token l%16, columns 4 (l/16) + e
  // (the records of the read-out O = Qg S + Bqk E hold Qg in place of Q' and,
  // in place of (Bqk U)^T, the A fragments of Bqk over tokens: token tile w,
  // token blocks pb <= w / 2, at bq_frag(w, pb))
  static constexpr size_t G = BU + (size_t)NT * 4 * 64 * 8;  // [D] fp32 e^G[C-1]
  static constexpr size_t BYTES = G + (size_t)D * 4;
};

// Fragment index of Bqk (token tile w, token block pb <= w / 2) in the BU
// region of a record of the Qg / Bqk read-out: six fragments of 1 KiB.
__device__ __forceinline__ int bq_frag(int w, int pb) { return (w < 2 ? w : 2 * w - 2) + pb; }

// LDS plan of the prep workgroup (bytes; two workgroups fit one CU).
//   region X: Kbar fragments of one stage of key blocks and the Kc^T
//             fragments; then L, T and L's diagonal blocks for the inverse;
//             then U (hi, lo) fragments
//   region Y: Kg^T and V^T fragments; -W fragments replace Kg^T
//   tile sums of log_alpha and beta
template <int D>
struct PrepLds {
  static constexpr int KB = D / 32, NT = D / 16;
  static constexpr int SB = KB < 2 ? KB : 2;   // key blocks per stage of A and Bqk
  static constexpr int PL = C + 4;             // fp32 row pitch of L and T
  static constexpr size_t KBAR = 0;                              // [hi,lo][wave][SB][64]
  static constexpr size_t KCT = KBAR + 2 * 4 * SB * FB;          // [NT][2][64] fp16
  static constexpr size_t XL = 0;                                // fp32 [C][PL]
  static constexpr size_t XT = XL + (size_t)C * PL * 4;          // fp32 [C][PL]
  static constexpr size_t XLD = XT + (size_t)C * PL * 4;         // fp32 [4][16][20]
  static constexpr size_t UX = 0;                                // [hi,lo][NT][2][64]
  static constexpr size_t XEND1 = KCT + NT * 2 * FB;
  static constexpr size_t XEND2 = XLD + 4 * 16 * 20 * 4;
  static constexpr size_t XEND3 = UX + 2 * NT * 2 * FB;
  static constexpr size_t XBYTES = XEND1 > XEND2 ? (XEND1 > XEND3 ? XEND1 : XEND3) : (XEND2 > XEND3 ? XEND2 : XEND3);
  static constexpr size_t KGT = XBYTES;                          // [NT][2][64]; later -W [NT][2][64]
  static constexpr size_t VT = KGT + NT * 2 * FB;                // [NT][2][64]
  static constexpr size_t TOT = VT + NT * 2 * FB;                // fp32 [4][D]
  static constexpr size_t BETA = TOT + (size_t)4 * D * 4;        // fp32 [C]
  static constexpr size_t EXPK = BETA + C * 4;                   // fp32 [2][D]: e^G[31], e^(G[C-1]-G[31])
  static constexpr size_t BYTES = EXPK + (size_t)2 * D * 4;
};

// Byte offset of element (token r of the wave's tile, column c4 + e) in a
// [NT column tiles][2 token blocks][64 lanes] fragment array whose fragments
// hold eight tokens of one column (the B operand of a product over tokens).
// Row layout: the lane holds token 16 w + l16 and columns c4 + e, c4 a
// multiple of 4.
__device__ __forceinline__ int tpos(int w, int l16, int c4, int e) {
  const int c = c4 + e;
  return ((((c >> 4) * 2 + (w >> 1)) * 64 + (c & 15) + 16 * (l16 >> 2)) * 16) + 2 * ((l16 & 3) + 4 * (w & 1));
}

template <int N>
__device__ __forceinline__ float row_shr(float v) {   // lane i of a DPP row gets lane i - N, 0 below the row
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + N, 0xF, 0xF, true));
}

// ---------------------------------------------------------------------------
// Kernel 1: per-chunk factors, one workgroup of four waves per (chunk slot,
// head).  Wave w holds tokens [16 w, 16 w + 16) of the chunk in "row layout":
// lane l has token 16 w + l % 16 and, for key block p, keys
// 32 p + kpos(l / 16, m), m = 0..7 -- which is at once the A operand of a
// product over keys and, lane for lane, the accumulator tiles of the
// transposed (key x token) matrix for key tiles 2p and 2p + 1.
// ---------------------------------------------------------------------------
// SCALAR: one gate per (token, head) instead of one per key channel; RAW: q,
// k unnormalised and beta a logit (normalised in the kernel).  Both are
// compile-time so that the input loads carry no branch.  QGB: the record
// carries Qg and Bqk for the read-out O = Qg S + Bqk E instead of Q' and
// (Bqk U)^T: no phase G, and 6 KiB of Bqk written in place of 16 KiB of
// (Bqk U)^T.
template <int D, bool SCALAR, bool RAW, bool QGB>
__device__ __forceinline__ void prep_item(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ log_alpha, const In* __restrict__ beta, int H, int h, int64_t t0, int len,
    unsigned char* __restrict__ rec, unsigned char* __restrict__ lds, int* __restrict__ status) {
  using R = Rec<D>;
  using L = PrepLds<D>;
  constexpr int KB = D / 32, NT = D / 16, SB = L::SB, PL = L::PL;
  const Rsrc rs = rec_rsrc(rec, R::BYTES);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, l16 = l & 15;
  const int r = 16 * w + l16;   // this lane's token in the chunk

  auto sKb = [&](int hl, int wv, int pb) { return reinterpret_cast<Frag*>(lds + L::KBAR) + ((hl * 4 + wv) * SB + pb) * 64; };
  float* sL = reinterpret_cast<float*>(lds + L::XL);
  float* sT = reinterpret_cast<float*>(lds + L::XT);
  float* sLdT = reinterpret_cast<float*>(lds + L::XLD);   // [4][16][20]
  float* sTot = reinterpret_cast<float*>(lds + L::TOT);
  float* sBeta = reinterpret_cast<float*>(lds + L::BETA);
  float* sExpK = reinterpret_cast<float*>(lds + L::EXPK);

  // ---- inputs in row layout --------------------------------------------------
  bf16x4 kr[KB][2], qr[KB][2], vr[KB][2];
  f32x4 gr[KB][2];
  float bt;
  {
    // every lane loads from a token clamped into the chunk and zeroes what
    // lies past its end afterwards: no load is conditional, so all of them
    // are in flight together
    const bool valid = r < len;
    const int64_t row = t0 + min(r, len - 1);
    const int64_t base = (row * H + h) * D;
    const bf16x4 z4 = bf16x4{(In)0.f, (In)0.f, (In)0.f, (In)0.f};
    // one gate per (token, head): the same log decay for every key channel
    float g1 = 0.f;
    if constexpr (SCALAR) g1 = log_alpha[row * H + h];
#pragma unroll
    for (int p = 0; p < KB; ++p)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int key = 32 * p + 16 * hh + 4 * g;
        const bf16x4 k1 = *reinterpret_cast<const bf16x4*>(k + base + key);
        const bf16x4 q1 = *reinterpret_cast<const bf16x4*>(q + base + key);
        const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(v + base + key);
        f32x4 g4;
        if constexpr (SCALAR) g4 = f32x4{g1, g1, g1, g1};
        else g4 = *reinterpret_cast<const f32x4*>(log_alpha + base + key);
        kr[p][hh] = valid ? k1 : z4;
        qr[p][hh] = valid ? q1 : z4;
        vr[p][hh] = valid ? v1 : z4;
        gr[p][hh] = valid ? g4 : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    const float b1 = (float)beta[row * H + h];
    bt = valid ? b1 : 0.f;
  }
  // raw inputs: unit q and k per token (the token's keys sit in lanes
  // l16 + 16 g, g = 0..3) and beta from its logit
  float rk = 1.f, rq = 1.f;
  if constexpr (RAW) {
    float ksq = 0.f, qsq = 0.f;
#pragma unroll
    for (int p = 0; p < KB; ++p)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k1 = (float)kr[p][hh][e], q1 = (float)qr[p][hh][e];
          ksq += k1 * k1;
          qsq += q1 * q1;
        }
    ksq += __shfl_xor(ksq, 16);
    ksq += __shfl_xor(ksq, 32);
    qsq += __shfl_xor(qsq, 16);
    qsq += __shfl_xor(qsq, 32);
    rk = inv_norm(ksq);
    rq = inv_norm(qsq);
    if (r < len) bt = sigmoid(bt);
  }

  // ---- A: cumulative log decay over the tokens ---------------------------------
  // inclusive scan over the 16 tokens of the tile (a DPP row), then the sums
  // of the earlier tiles from LDS
#pragma unroll
  for (int p = 0; p < KB; ++p)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = gr[p][hh][e];
        x += row_shr<1>(x);
        x += row_shr<2>(x);
        x += row_shr<4>(x);
        x += row_shr<8>(x);
        gr[p][hh][e] = x;
      }
  if (l16 == 15) {
#pragma unroll
    for (int p = 0; p < KB; ++p)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        *reinterpret_cast<f32x4*>(sTot + w * D + 32 * p + 16 * hh + 4 * g) = gr[p][hh];
  }
  if (g == 0) sBeta[r] = bt;
  __syncthreads();

  f32x4 gmv[KB][2];   // G[31] of this lane's keys
#pragma unroll
  for (int p = 0; p < KB; ++p)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int key = 32 * p + 16 * hh + 4 * g;
      f32x4 t[4];
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) t[wv] = *reinterpret_cast<const f32x4*>(sTot + wv * D + key);
      f32x4 off = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int wv = 0; wv < 3; ++wv)
        if (wv < w) off += t[wv];
      gr[p][hh] += off;
      gmv[p][hh] = t[0] + t[1];
    }
  // per-key exponentials, once per key: e^G[31] and e^G[C-1] (threads 0..D-1),
  // e^(G[C-1] - G[31]) (threads D..2D-1)
  {
    const int key = tid % D;
    const float tm = sTot[key] + sTot[D + key];
    const float tc = tm + sTot[2 * D + key] + sTot[3 * D + key];
    if (tid < D) {
      sExpK[key] = __expf(tm);
      st_rec<float>(rs, R::G + 4 * key, __expf(tc));
    } else if (tid < 2 * D) {
      sExpK[D + key] = __expf(tc - tm);
    }
  }
  __syncthreads();

  // ---- B: decay-scaled operands --------------------------------------------------
  //   X = e^(G - G[31]);  Ka = K X, Kbar = K / X, Qa = Q X  (anchored at token 31)
  //   Kg = K e^G, Qg = Q e^G, Kc = K e^(G[C-1] - G)
  Frag kaF[KB], kbH[KB], kbL[KB], qaH[KB], qaL[KB];
  float qg[KB][8];
  float dgmax = 0.f;   // largest |G - G[31]|: e^(+-80) is the most the factors may span
#pragma unroll
  for (int p = 0; p < KB; ++p)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int key = 32 * p + 16 * hh + 4 * g;
      const f32x4 egm4 = *reinterpret_cast<const f32x4*>(sExpK + key);
      const f32x4 ecm4 = *reinterpret_cast<const f32x4*>(sExpK + D + key);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * hh + e;
        const float gm = gmv[p][hh][e];
        const float dg = gr[p][hh][e] - gm;
        dgmax = fmaxf(dgmax, fabsf(dg));
        const float x = __expf(dg), ix = __expf(-dg);
        const float egm = egm4[e], ecm = ecm4[e];
        const float kx = (float)kr[p][hh][e] * rk, qx = (float)qr[p][hh][e] * rq;
        const float ka = kx * x, kb = kx * ix, qa = qx * x;
        kaF[p][m] = (In)ka;
        kbH[p][m] = (In)kb;
        kbL[p][m] = (In)(kb - (float)kbH[p][m]);
        qaH[p][m] = (In)qa;
        qaL[p][m] = (In)(qa - (float)qaH[p][m]);
        qg[p][m] = qa * egm;
        const int pos = tpos(w, l16, 32 * p + 16 * hh + 4 * g, e);
        *reinterpret_cast<In*>(lds + L::KGT + pos) = (In)(ka * egm);
        *reinterpret_cast<_Float16*>(lds + L::KCT + pos) = (_Float16)(kb * ecm);
        *reinterpret_cast<In*>(lds + L::VT + pos) = vr[p][hh][e];
      }
    }
#pragma unroll
  for (int pb = 0; pb < SB; ++pb) {
    sKb(0, w, pb)[l] = kbH[pb];
    sKb(1, w, pb)[l] = kbL[pb];
  }
  // a gate sum beyond the fp32 exponent range: report it (results of this
  // chunk may be non-finite)
  if (__any(dgmax > kMaxAnchoredExp) && l == 0)
    __hip_atomic_fetch_or(status, kStatusGateRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();

  // ---- C: A = Ka Kbar^T (tiles (w, j)) and Bqk^T = Kbar Qa^T (tiles (j, w)),
  //      j <= w, in stages of SB key blocks; Kc^T fragments to the record ----
  for (int i = tid; i < NT * 2 * 64; i += kPrepThreads)
    st_rec<HFrag>(rs, R::KC + 16 * (size_t)i, reinterpret_cast<const HFrag*>(lds + L::KCT)[i]);
  f32x4 accA[4], accB[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) accA[j] = accB[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KB / SB; ++s) {
    if (s > 0) {
      __syncthreads();   // every wave is done with the previous stage
#pragma unroll
      for (int pb = 0; pb < SB; ++pb) {
        sKb(0, w, pb)[l] = kbH[s * SB + pb];
        sKb(1, w, pb)[l] = kbL[s * SB + pb];
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j > w) break;
#pragma unroll
      for (int pb = 0; pb < SB; ++pb) {
        const int p = s * SB + pb;
        const Frag bh = sKb(0, j, pb)[l];   // this wave's own fragments too: no
        const Frag bl = sKb(1, j, pb)[l];   // register/LDS select per tile
        mma(accA[j], kaF[p], bh);
        mma(accB[j], bh, qaH[p]);
        mma(accB[j], bh, qaL[p]);
        mma(accB[j], bl, qaH[p]);
      }
    }
  }
  // Bqk as the A operand over tokens (rows: this wave's tokens), split; the
  // Bqk^T tiles (j, w) are, lane for lane, its fragments
  Frag bqH[2], bqL[2];
  HFrag bqF[2];   // single fp16, for a Qg / Bqk record
#pragma unroll
  for (int pb = 0; pb < 2; ++pb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int j = 2 * pb + hf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = (j < w || (j == w && 4 * g + e <= l16)) ? accB[j][e] : 0.f;
        const In hv = (In)x;
        bqH[pb][4 * hf + e] = hv;
        bqL[pb][4 * hf + e] = (In)(x - (float)hv);
        bqF[pb][4 * hf + e] = (_Float16)x;
      }
    }
  if constexpr (QGB) {
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
      if (pb <= (w >> 1)) st_rec<HFrag>(rs, R::BU + ((size_t)bq_frag(w, pb) * 64 + l) * 16, bqF[pb]);
#pragma unroll
    for (int p = 0; p < KB; ++p) {
      HFrag qh;
#pragma unroll
      for (int m = 0; m < 8; ++m) qh[m] = (_Float16)qg[p][m];
      st_rec<HFrag>(rs, R::QP + ((w * KB + p) * 64 + l) * 16, qh);
    }
  }
  __syncthreads();   // region X is reused for L and T

  // ---- D: T = (I + L)^-1, L = Diag(beta) A strictly lower ---------------------
  {
    f32x4 brow;
#pragma unroll
    for (int e = 0; e < 4; ++e) brow[e] = sBeta[16 * w + 4 * g + e];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j > w) break;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = 16 * w + 4 * g + e, jj = 16 * j + l16;
        const float lv = (jj < rr) ? brow[e] * accA[j][e] : 0.f;
        sL[rr * PL + jj] = lv;
        if (j == w) sLdT[(w * 16 + l16) * 20 + 4 * g + e] = lv;   // column jj of the block as a row
      }
    }
  }
  __syncthreads();
  // 16 x 16 diagonal blocks by column-oriented forward substitution (wave 0,
  // lane = (block, column)), then block doubling
  //   [[X, 0], [Y, Z]]^-1 = [[X^-1, 0], [-Z^-1 Y X^-1, Z^-1]]
  // for the 16-blocks (1,0), (3,2) and then the 32-block (1,0).  The block
  // products run on v_mfma_f32_16x16x4_f32 with the reduction index of
  // instruction s taken as 4 g + s: a row of the left factor is one 16-byte
  // LDS read and the right factor is an accumulator tile.
  if (w == 0) {
    const int bk = l >> 4, cc = l & 15;
    float x[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) x[rr] = (rr == cc) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      f32x4 colj[4];
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) colj[qd] = *reinterpret_cast<const f32x4*>(sLdT + (bk * 16 + j) * 20 + 4 * qd);
#pragma unroll
      for (int rr = j + 1; rr < 16; ++rr) x[rr] -= colj[rr >> 2][rr & 3] * x[j];
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) sT[(16 * bk + rr) * PL + 16 * bk + cc] = x[rr];
  }
  __syncthreads();
  const int c = l16;
  auto ctile = [&](int Rb, int Kb) {
    f32x4 t;
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = sT[(16 * Rb + 4 * g + e) * PL + 16 * Kb + c];
    return t;
  };
  auto mma_rows = [&](f32x4& acc, const float* M, int Rb, int Kb, const f32x4& b) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(M + (16 * Rb + l16) * PL + 16 * Kb + 4 * g);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s4], b[s4], acc, 0, 0, 0);
  };
  if (w < 2) {   // T(bb, a) = -T(bb, bb) L(bb, a) T(a, a), bb = a + 1
    const int a = 2 * w, bb = a + 1;
    f32x4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
    mma_rows(y, sL, bb, a, ctile(a, a));
    mma_rows(z, sT, bb, bb, y);
#pragma unroll
    for (int e = 0; e < 4; ++e) sT[(16 * bb + 4 * g + e) * PL + 16 * a + c] = -z[e];
  }
  __syncthreads();
  float* sScr = sLdT;   // the diagonal blocks are done with: Y tiles [4][16][20]
  {   // Y = L[32:64, 0:32] T[0:32, 0:32]; wave w owns 16-tile (bi, bj)
    const int bi = w >> 1, bj = w & 1;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    for (int kb = bj; kb < 2; ++kb) mma_rows(y, sL, 2 + bi, kb, ctile(kb, bj));
#pragma unroll
    for (int e = 0; e < 4; ++e) sScr[(w * 16 + 4 * g + e) * 20 + c] = y[e];
  }
  __syncthreads();
  {   // T[32:64, 0:32] = -T[32:64, 32:64] Y
    const int bi = w >> 1, bj = w & 1;
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb <= bi; ++kb) {
      f32x4 yt;
#pragma unroll
      for (int e = 0; e < 4; ++e) yt[e] = sScr[((2 * kb + bj) * 16 + 4 * g + e) * 20 + c];
      mma_rows(z, sT, 2 + bi, 2 + kb, yt);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) sT[(32 + 16 * bi + 4 * g + e) * PL + 16 * bj + c] = -z[e];
  }
  __syncthreads();
  // T' = T Diag(beta), this wave's rows, as A fragments over token blocks
  Frag tf[2];
#pragma unroll
  for (int pb = 0; pb < 2; ++pb)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int j = 32 * pb + kpos(g, m);
      tf[pb][m] = (In)((j <= r) ? sT[r * PL + j] * sBeta[j] : 0.f);
    }

  // ---- E: W = T' Kg (tiles (w, it)) and W^T (tiles (it, w)) -> record W -----
  const int npb = (w >> 1) + 1;   // token blocks with T'[r][j] != 0
  Half wneg[NT];
  HFrag wrec;   // two key tiles of W, stored as one fragment
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    f32x4 wc = {0.f, 0.f, 0.f, 0.f}, wt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      if (pb >= npb) break;
      const Frag kg = reinterpret_cast<const Frag*>(lds + L::KGT)[(it * 2 + pb) * 64 + l];
      mma(wc, tf[pb], kg);
      mma(wt, kg, tf[pb]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wrec[4 * (it & 1) + e] = (_Float16)wt[e];
      wneg[it][e] = (In)(-wc[e]);
    }
    if (it & 1)
      st_rec<HFrag>(rs, R::W + ((w * KB + (it >> 1)) * 64 + l) * 16, wrec);
  }
  __syncthreads();   // Kg^T and T are no longer read

  // ---- F: -W tiles to LDS (A operand of W^T over tokens); U = T' V -> record,
  //      and U split to LDS (B operand over tokens); a Qg / Bqk record needs
  //      only U -----------------------------------------------------------------
  if constexpr (!QGB) {
#pragma unroll
    for (int it = 0; it < NT; ++it)
      *reinterpret_cast<Half*>(lds + L::KGT + ((it * 2 + (w >> 1)) * 64 + l) * 16 + 8 * (w & 1)) = wneg[it];
  }
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    f32x4 uc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      if (pb >= npb) break;
      mma(uc, tf[pb], reinterpret_cast<const Frag*>(lds + L::VT)[(ct * 2 + pb) * 64 + l]);
    }
    HHalf u16;
#pragma unroll
    for (int e = 0; e < 4; ++e) u16[e] = (_Float16)uc[e];
    st_rec<HHalf>(rs, R::U + ((ct * 4 + w) * 64 + l) * 8, u16);
    if constexpr (!QGB) {
      Half uh, ul;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uh[e] = (In)uc[e];
        ul[e] = (In)(uc[e] - (float)uh[e]);
      }
      const size_t off = ((ct * 2 + (w >> 1)) * 64 + l) * 16 + 8 * (w & 1);
      *reinterpret_cast<Half*>(lds + L::UX + off) = uh;
      *reinterpret_cast<Half*>(lds + L::UX + NT * 2 * FB + off) = ul;
    }
  }
  if constexpr (QGB) return;
  __syncthreads();

  // ---- G: Q'^T = Qg^T - W^T Bqk^T (tiles (it, w)) -> record Q';
  //      (Bqk U)^T (tiles (ct, w)) -> record ----------------------------------------
  HFrag qrec;   // two key tiles of Q', stored as one fragment
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    f32x4 acc;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = qg[it >> 1][4 * (it & 1) + e];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      if (pb >= npb) break;
      const Frag wa = reinterpret_cast<const Frag*>(lds + L::KGT)[(it * 2 + pb) * 64 + l];
      mma(acc, wa, bqH[pb]);
      mma(acc, wa, bqL[pb]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) qrec[4 * (it & 1) + e] = (_Float16)acc[e];
    if (it & 1)
      st_rec<HFrag>(rs, R::QP + ((w * KB + (it >> 1)) * 64 + l) * 16, qrec);
  }
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    f32x4 bu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      if (pb >= npb) break;
      const Frag uh = reinterpret_cast<const Frag*>(lds + L::UX)[(ct * 2 + pb) * 64 + l];
      const Frag ul = reinterpret_cast<const Frag*>(lds + L::UX + NT * 2 * FB)[(ct * 2 + pb) * 64 + l];
      mma(bu, uh, bqH[pb]);   // operands swapped: the tile of (Bqk U)^T
      mma(bu, ul, bqH[pb]);
      mma(bu, uh, bqL[pb]);
    }
    HHalf bu16;
#pragma unroll
    for (int e = 0; e < 4; ++e) bu16[e] = (_Float16)bu[e];
    st_rec<HHalf>(rs, R::BU + ((ct * 4 + w) * 64 + l) * 8, bu16);
  }
}

// One (chunk slot, head) item of the two-kernel path: slots in reverse
// order, so that the state pass, which starts from each sequence's first
// chunk, finds those records -- written last -- in the memory-side cache.
template <int D, bool SCALAR, bool RAW>
__global__ __launch_bounds__(kPrepThreads, 2) void prep_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ log_alpha, const In* __restrict__ beta, const int32_t* __restrict__ cu,
    int N, int H, unsigned char* __restrict__ ws, int* __restrict__ status) {
  __shared__ __align__(16) unsigned char lds[PrepLds<D>::BYTES];
  const int64_t item = blockIdx.x;
  const int64_t slot = (int64_t)(gridDim.x / H) - 1 - item / H;
  const int h = (int)(item % H);
  int n, len;
  int64_t t0;
  if (!decode_slot(cu, N, slot, n, t0, len)) return;   // whole workgroup: unused slot
  prep_item<D, SCALAR, RAW, false>(q, k, v, log_alpha, beta, H, h, t0, len,
                                   ws + ((size_t)slot * H + h) * Rec<D>::BYTES, lds, status);
}

// ---------------------------------------------------------------------------
// Sequential pass over the chunks of one (sequence, head) for a slice of VT
// value tiles (16 VT columns) of S.  Wave w owns key rows [D/4 w, D/4 (w+1))
// of the slice as accumulators and token tile w of every chunk; the operands
// of the next two chunks are in flight while the current one is computed.
// W, Q' (or Qg) and Kc serve every value tile of the slice, so a wider slice loads
// them once for more columns.
// ---------------------------------------------------------------------------
template <int D, int VT, bool QGB>
struct Ops {
  static constexpr int KB = D / 32, KTW = D / 64;
  HFrag w[KB];               // W, token tile of this wave
  HFrag qp[KB];              // Q' (or Qg), token tile of this wave
  HFrag kc[KTW][2];          // Kc^T for this wave's key tiles
  HHalf u[VT];               // U, token tile of this wave, the slice's value tiles
  HHalf bu[QGB ? 1 : VT];    // (Bqk U)^T, same tiles
  HFrag bq[QGB ? 2 : 1];     // Bqk over tokens, two token blocks (tiles 0, 1: the second is zero)
  f32x4 gam[KTW];            // e^G[C-1] for this lane's key rows
};

// The operand loads of one chunk, in three parts that the step spreads over
// its phases so that the vector memory path works while the MFMAs do.
template <int D, int VT, bool QGB>
__device__ __forceinline__ void load_ops_part(Ops<D, VT, QGB>& o, Rsrc rs, int part, int w, int l, int g, int vt0) {
  using R = Rec<D>;
  using O = Ops<D, VT, QGB>;
  if (part == 0) {
#pragma unroll
    for (int p = 0; p < O::KB; ++p) o.w[p] = ld_rec<HFrag>(rs, R::W + ((w * O::KB + p) * 64 + l) * 16);
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      o.u[t] = ld_rec<HHalf>(rs, R::U + (((vt0 + t) * 4 + w) * 64 + l) * 8);
      if constexpr (!QGB) o.bu[t] = ld_rec<HHalf>(rs, R::BU + (((vt0 + t) * 4 + w) * 64 + l) * 8);
    }
    if constexpr (QGB) {
      // waves 0 and 1 have one block: their second fragment is zero, so
      // that the read-out's products take no branch (a product under a
      // lane mask would still run on every lane)
      o.bq[0] = ld_rec<HFrag>(rs, R::BU + ((size_t)bq_frag(w, 0) * 64 + l) * 16);
      const HFrag b1 = ld_rec<HFrag>(rs, R::BU + ((size_t)bq_frag(w, w >> 1) * 64 + l) * 16);
#pragma unroll
      for (int m = 0; m < 8; ++m) o.bq[1][m] = w >= 2 ? b1[m] : (_Float16)0.f;
    }
  } else if (part == 1) {
#pragma unroll
    for (int p = 0; p < O::KB; ++p) o.qp[p] = ld_rec<HFrag>(rs, R::QP + ((w * O::KB + p) * 64 + l) * 16);
  } else {
#pragma unroll
    for (int kt = 0; kt < O::KTW; ++kt)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int kti = w * O::KTW + kt;
        o.kc[kt][p] = ld_rec<HFrag>(rs, R::KC + ((kti * 2 + p) * 64 + l) * 16);
      }
#pragma unroll
    for (int kt = 0; kt < O::KTW; ++kt)
      o.gam[kt] = ld_rec<f32x4>(rs, R::G + (16 * (w * O::KTW + kt) + 4 * g) * 4);
  }
}

template <int D, int VT, bool QGB>
__device__ __forceinline__ void load_ops(Ops<D, VT, QGB>& o, Rsrc rs, int w, int l, int g, int vt0) {
#pragma unroll
  for (int part = 0; part < 3; ++part) load_ops_part<D, VT, QGB>(o, rs, part, w, l, g, vt0);
}

// Chunk-ready flags of the one-launch path: flag[slot * H + h] turns nonzero
// once the record of (slot, h) is complete.  A wait gives up after about two
// seconds (the whole prep of a million-token sequence takes milliseconds),
// sets the status word and lets the pass run on with NaN outputs, so that no
// wave can hang.
constexpr int kSpinLimit = 1 << 21;
constexpr int kLeadSpinLimit = 1 << 18;   // a prep item's wait for the pass to come within reach

struct Sync {
  const int* flags;   // nullptr: records are complete before the pass starts
  int* status;
  int* marks;         // non-null: set flag (slot, head) to kConsumed after each chunk step
};

// Flag value of a chunk whose step the state pass (its first value slice)
// has finished; prep items that may run only a bounded number of chunks
// ahead of the pass wait for it (any nonzero flag means published).
constexpr int kConsumed = 2;

// Readiness of the records a pass is about to load.  `upto` is the last
// chunk known to be published, every earlier one included.  When chunk c is
// needed beyond it, lane i polls chunk upto + 1 + i % 16 (clamped to the
// last chunk) and `upto` advances over the published run that starts right
// after it, until it reaches c.  (A run that started at c itself would say
// nothing of the chunks between: chunks are published out of order.)  A
// pass that trails the prep by more than 16 chunks thus polls once every 16
// steps, and one right behind it polls every step.  The acquire fence keeps
// the record loads after the poll.
__device__ __forceinline__ void need_record(const Sync& sy, int64_t slot0, int H, int h, int c, int nch, int lane,
                                            int& upto, bool& failed) {
  if (!sy.flags || failed || c <= upto) return;
  for (int spin = 0;; ++spin) {
    const int first = upto + 1;
    const int* f = sy.flags + (slot0 + min(first + (lane & 15), nch - 1)) * H + h;
    const int ready = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t mask = __ballot(ready != 0) & 0xFFFFull;
    upto = first + __builtin_ctzll(~mask) - 1;   // chunks first .. upto are published
    if (upto >= c) break;
    if (spin >= kSpinLimit) {
      failed = true;
      if (lane == 0) __hip_atomic_fetch_or(sy.status, kStatusWaitGaveUp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// LDS of the state pass: S and E as B operands; S twice (by chunk parity)
// when the read-out reads it again after the second barrier of a step.
template <int D, int VT, bool HOLD_SF>
struct StateLds {
  static constexpr int KB = D / 32;
  static constexpr size_t SB = (size_t)VT * KB * 64 * 16;        // one copy of S: HFrag [VT][KB][64]
  static constexpr size_t S = 0;
  static constexpr size_t E = S + (HOLD_SF ? 1 : 2) * SB;         // HFrag [VT][2][64]
  static constexpr size_t BYTES = E + (size_t)VT * 2 * 64 * 16;
};

// The pass of (sequence n, head h, value slice vt).  NB operand buffers in
// rotation (3: chunks c+1 and c+2 in flight during step c; 2: chunk c+1).
// HOLD_SF keeps this step's S fragments in registers for both products;
// otherwise the read-out reads them from LDS again, from a copy that the
// next step does not overwrite.  Both give the same results bit for bit.
template <int D, int VT, int NB, bool HOLD_SF, bool QGB>
__device__ __forceinline__ void state_task(const int32_t* __restrict__ cu, int H, const float* init, float* fin,
                                           In* __restrict__ o, const unsigned char* __restrict__ ws,
                                           const int32_t* __restrict__ sidx, int pool_slots, int n, int h, int vt,
                                           const Sync& sy, unsigned char* __restrict__ lds) {
  static_assert(NB == 2 || NB == 3, "two or three operand buffers");
  using R = Rec<D>;
  using SL = StateLds<D, VT, HOLD_SF>;
  constexpr int KB = D / 32, KTW = D / 64;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
  const int vt0 = vt * VT;   // first value tile of the slice
  const int64_t bos = cu[n], eos = cu[n + 1];
  const int nch = (int)((eos - bos + kChunk - 1) / kChunk);
  const int64_t slot0 = bos / kChunk + n;

  HFrag (*sE)[2][64] = reinterpret_cast<HFrag (*)[2][64]>(lds + SL::E);   // E as the B operand
  auto sS = [&](int c) {   // S as the B operand
    return reinterpret_cast<HFrag (*)[KB][64]>(lds + SL::S + (HOLD_SF ? 0 : (c & 1) * SL::SB));
  };

  const int64_t sslot = state_slot(sidx, pool_slots, n);
  if (sslot < 0) init = nullptr, fin = nullptr;
  const int64_t sbase = (sslot * H + h) * D;   // row (value channel) base of state[slot][h]
  f32x4 S[VT][KTW];
#pragma unroll
  for (int t = 0; t < VT; ++t)
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int kti = w * KTW + kt, col = 16 * (vt0 + t) + l16;
      S[t][kt] = init ? *reinterpret_cast<const f32x4*>(init + (sbase + col) * D + 16 * kti + 4 * g)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // The initial state is in registers before any record load is issued: a
  // load still in flight into S at the loop head would make the compiler
  // wait there for every load, at every iteration.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  auto rec_of = [&](int c) {
    return rec_rsrc(ws + ((size_t)(slot0 + min(c, nch - 1)) * H + h) * R::BYTES, R::BYTES);
  };
  bool failed = false;   // a wait for records gave up: outputs and final state become NaN
  int upto = -1;          // last chunk whose record is known to be published

  // one chunk step with operands `ops`; meanwhile the operands of a later
  // chunk (record `nrs`) are loaded into `nxt`, one part per phase, once
  // the records up to chunk `need` are known to be published (need < 0:
  // an earlier step made sure of it)
  auto step = [&](const Ops<D, VT, QGB>& ops, int c, Ops<D, VT, QGB>& nxt, Rsrc nrs, int need) {
    if (need >= 0) need_record(sy, slot0, H, h, need, nch, l, upto, failed);
    load_ops_part<D, VT, QGB>(nxt, nrs, 0, w, l, g, vt0);
    const int64_t t0 = bos + (int64_t)c * kChunk;
    const int len = (int)min<int64_t>(kChunk, eos - t0);
    HFrag (*sSc)[KB][64] = sS(c);
#pragma unroll
    for (int t = 0; t < VT; ++t)
#pragma unroll
      for (int kt = 0; kt < KTW; ++kt) {
        const int kti = w * KTW + kt;
        HHalf hs;
#pragma unroll
        for (int e = 0; e < 4; ++e) hs[e] = (_Float16)S[t][kt][e];
        *reinterpret_cast<HHalf*>(reinterpret_cast<_Float16*>(&sSc[t][kti >> 1][l]) + 4 * (kti & 1)) = hs;
      }
    __syncthreads();
    load_ops_part<D, VT, QGB>(nxt, nrs, 1, w, l, g, vt0);
    // token tile w: W S first -- E gates the other waves; Q' S only after
    // the state update has been issued
    HFrag sf[HOLD_SF ? VT : 1][KB];
    if constexpr (HOLD_SF) {
#pragma unroll
      for (int t = 0; t < VT; ++t)
#pragma unroll
        for (int p = 0; p < KB; ++p) sf[t][p] = sSc[t][p][l];
    }
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      f32x4 wsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < KB; ++p) mma(wsum, ops.w[p], HOLD_SF ? sf[HOLD_SF ? t : 0][p] : sSc[t][p][l]);
      // E = U - W S, published as the B operand over tokens
      HHalf eh;
#pragma unroll
      for (int e = 0; e < 4; ++e) eh[e] = (_Float16)((float)ops.u[t][e] - wsum[e]);
      *reinterpret_cast<HHalf*>(reinterpret_cast<_Float16*>(&sE[t][w >> 1][l]) + 4 * (w & 1)) = eh;
    }
    __syncthreads();
    load_ops_part<D, VT, QGB>(nxt, nrs, 2, w, l, g, vt0);
    // S <- Diag(e^G[C-1]) S + Kc^T E
#pragma unroll
    for (int t = 0; t < VT; ++t)
#pragma unroll
      for (int kt = 0; kt < KTW; ++kt) {
        S[t][kt] *= ops.gam[kt];
#pragma unroll
        for (int p = 0; p < 2; ++p) mma(S[t][kt], ops.kc[kt][p], sE[t][p][l]);
      }
    // O^T = S^T Q'^T + (Bqk U)^T for token tile w, off the state's
    // dependency chain.  The operands swapped in the product give the
    // transposed tile: lane l holds token 16 w + l % 16 and four adjacent
    // value columns, stored as one 8-byte write.
    const int r = 16 * w + l16;
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      f32x4 ot;
      if constexpr (QGB) {
        // O^T = S^T Qg^T + E^T Bqk^T: E of this chunk is still in LDS
        ot = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) mma(ot, sE[t][pb][l], ops.bq[pb]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ot[e] = (float)ops.bu[t][e];
      }
#pragma unroll
      for (int p = 0; p < KB; ++p) mma(ot, HOLD_SF ? sf[HOLD_SF ? t : 0][p] : sSc[t][p][l], ops.qp[p]);
      Half ob;
#pragma unroll
      for (int e = 0; e < 4; ++e) ob[e] = (In)(failed ? __builtin_nanf("") : ot[e]);
      if (r < len) *reinterpret_cast<Half*>(o + ((t0 + r) * H + h) * D + 16 * (vt0 + t) + 4 * g) = ob;
    }
    if (sy.marks && tid == 0)
      __hip_atomic_store(sy.marks + (slot0 + c) * H + h, kConsumed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // Operand buffers in rotation: while chunk c is computed, the operands of
  // the next NB - 1 chunks are in flight (past the last chunk the last
  // record is read again, so every step issues the same loads and the
  // compiler's waits stay exact).  Twelve steps per loop iteration, a
  // multiple of NB, so that the buffers hold the same roles at every loop
  // head; the iterations have no early exit, and the last nch % 12 chunks
  // run after the loop: an exit edge into the loop's latch would make the
  // compiler wait there for every load in flight.  The one-launch path
  // checks that a record is published before the step that loads it; in the
  // loop the last step of an iteration checks one chunk further for the
  // first step of the next, so that no wait for the producers sits at the
  // loop head (the compiler then drains every load in flight there too).
  Ops<D, VT, QGB> bufA, bufB, bufC;
  if (nch > 0) {
    need_record(sy, slot0, H, h, 0, nch, l, upto, failed);
    load_ops<D, VT, QGB>(bufA, rec_of(0), w, l, g, vt0);
    if constexpr (NB == 3) {
      need_record(sy, slot0, H, h, 1, nch, l, upto, failed);
      load_ops<D, VT, QGB>(bufB, rec_of(1), w, l, g, vt0);
    }
    need_record(sy, slot0, H, h, NB - 1, nch, l, upto, failed);   // for the first step
  }
  // step u of 12 in a loop iteration: the chunk to check before its loads
  auto need_of = [&](int c, int u) { return u == 0 ? -1 : c + NB - 1 + (u == 11); };
  int c0 = 0;
  for (; c0 + 12 <= nch; c0 += 12) {
    if constexpr (NB == 3) {
#pragma unroll
      for (int u = 0; u < 12; u += 3) {
        step(bufA, c0 + u, bufC, rec_of(c0 + u + 2), need_of(c0 + u, u));
        step(bufB, c0 + u + 1, bufA, rec_of(c0 + u + 3), need_of(c0 + u + 1, u + 1));
        step(bufC, c0 + u + 2, bufB, rec_of(c0 + u + 4), need_of(c0 + u + 2, u + 2));
      }
    } else {
#pragma unroll
      for (int u = 0; u < 12; u += 2) {
        step(bufA, c0 + u, bufB, rec_of(c0 + u + 1), need_of(c0 + u, u));
        step(bufB, c0 + u + 1, bufA, rec_of(c0 + u + 2), need_of(c0 + u + 1, u + 1));
      }
    }
  }
  if constexpr (NB == 3) {
#pragma unroll
    for (int u = 0; u < 12; u += 3) {
      const int c = c0 + u;
      if (c >= nch) break;
      step(bufA, c, bufC, rec_of(c + 2), c + 2);
      if (c + 1 >= nch) break;
      step(bufB, c + 1, bufA, rec_of(c + 3), c + 3);
      if (c + 2 >= nch) break;
      step(bufC, c + 2, bufB, rec_of(c + 4), c + 4);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 12; u += 2) {
      const int c = c0 + u;
      if (c >= nch) break;
      step(bufA, c, bufB, rec_of(c + 1), c + 1);
      if (c + 1 >= nch) break;
      step(bufB, c + 1, bufA, rec_of(c + 2), c + 2);
    }
  }

  // The last steps loaded records past the end that are never used.  Wait
  // for them here, once per pass: left in flight, they would make the
  // compiler wait for every load at each loop head of the next pass that
  // this workgroup runs.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  if (fin) {
#pragma unroll
    for (int t = 0; t < VT; ++t)
#pragma unroll
      for (int kt = 0; kt < KTW; ++kt) {
        const int kti = w * KTW + kt, col = 16 * (vt0 + t) + l16;
        const float nanv = __builtin_nanf("");
        *reinterpret_cast<f32x4*>(fin + (sbase + col) * D + 16 * kti + 4 * g) =
            failed ? f32x4{nanv, nanv, nanv, nanv} : S[t][kt];
      }
  }
}

// Task index -> (sequence-head pair, value slice).  Tasks below nstatic (a
// multiple of 8 NV) are dealt so that the NV slices of one (sequence, head)
// share an XCD (and its L2), since workgroups are dealt to the 8 XCDs
// round-robin and the first such block index is a multiple of 8; they cover
// the pairs below nstatic / NV.  Later tasks go in pair order.
template <int NV>
__device__ __forceinline__ void task_of(int task, int nstatic, int& pair, int& vt) {
  if (task < nstatic) {
    const int xcd = task & 7, rest = task >> 3;
    vt = rest % NV;
    pair = (rest / NV) * 8 + xcd;
  } else {
    vt = task % NV;
    pair = task / NV;
  }
}

// Two-kernel path, kernel 2: one workgroup per (sequence, head, slice),
// one workgroup per CU (the pass is bound by the operand bytes a CU keeps in
// flight, and a second workgroup on the same CU lowers the throughput of
// both when a batch has more workgroups than CUs).
template <int D, int VT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void state_kernel(
    const int32_t* __restrict__ cu, int N, int H, const float* init, float* fin, In* __restrict__ o,
    const unsigned char* __restrict__ ws, const int32_t* __restrict__ sidx, int pool_slots) {
  constexpr int NV = D / (16 * VT);
  __shared__ __align__(16) unsigned char lds[StateLds<D, VT, true>::BYTES];
  int pair, vt;
  task_of<NV>(blockIdx.x, gridDim.x, pair, vt);
  if (pair >= N * H) return;
  state_task<D, VT, 3, true, false>(cu, H, init, fin, o, ws, sidx, pool_slots, pair / H, pair % H, vt,
                                    Sync{nullptr, nullptr, nullptr}, lds);
}

// ---------------------------------------------------------------------------
// One-launch path: the prep and the state pass in one grid, so that the pass
// follows the prep chunk by chunk instead of waiting for all of it, and the
// CUs it leaves idle (a long sequence with few heads has few slices) run the
// prep meanwhile.
//   blocks [0, nstate):     state tasks, the first ones dealt statically,
//                           then from a ticket;
//   blocks [nstate, grid):  one prep item (chunk slot, head) each, in slot
//                           order; its flag publishes its record.
// Prep blocks wait for nothing, and the state blocks are at most a quarter
// of the blocks the device holds at once, so prep blocks always find room
// and every awaited record is eventually published, in whatever order the
// blocks are dispatched.
// Header words in the workspace: [0] state ticket, [1] status (bits
// kStatus*); zeroed with the flags before each call.
// ---------------------------------------------------------------------------
struct FusedHdr {
  int state_ticket, status, pad[62];
};

__global__ void fused_init_kernel(int* __restrict__ flags, int64_t nflags, FusedHdr* __restrict__ hdr) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = i; j < nflags; j += stride) flags[j] = 0;
  if (i == 0) hdr->state_ticket = hdr->status = 0;
}

// The state role of the one-launch kernel shares the prep's register budget
// (two blocks per CU): one-tile slices keep three operand buffers and hold
// S's fragments; wider slices keep two and read S again from LDS.
template <int VT>
struct FusedState {
  static constexpr int NB = VT == 1 ? 3 : 2;
  static constexpr bool HOLD_SF = VT == 1;
  // the shorter Qg / Bqk record where the prep is the longer leg (many
  // (sequence, head) pairs); one-tile slices, chosen when the pass is the
  // longer leg, keep Q' and (Bqk U)^T, whose read-out loads and multiplies
  // less per step
  static constexpr bool QGB = VT >= 2;
};

__global__ void clear_status_kernel(int* status) {
  if (threadIdx.x == 0) *status = 0;
}

template <int D, int VT>
struct FusedLds {
  using SL = StateLds<D, VT, FusedState<VT>::HOLD_SF>;
  static constexpr size_t BYTES = PrepLds<D>::BYTES > SL::BYTES ? PrepLds<D>::BYTES : SL::BYTES;
};

template <int D, bool SCALAR, bool RAW, int VT>
__global__ __launch_bounds__(kPrepThreads, 2) void fused_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ log_alpha, const In* __restrict__ beta, const int32_t* __restrict__ cu,
    int N, int H, const float* init, float* fin, In* __restrict__ o, unsigned char* __restrict__ ws,
    int* __restrict__ flags, FusedHdr* __restrict__ hdr, const int32_t* __restrict__ sidx, int pool_slots,
    int nstate, int ntot, int lead) {
  constexpr int NV = D / (16 * VT);
  __shared__ __align__(16) unsigned char lds[FusedLds<D, VT>::BYTES];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= nstate) {
    const int64_t item = (int64_t)blockIdx.x - nstate;
    const int64_t slot = item / H;
    const int h = (int)(item % H);
    int n, len;
    int64_t t0;
    if (!decode_slot(cu, N, slot, n, t0, len)) return;   // whole workgroup: unused slot
    if (lead > 0 && t0 - cu[n] >= (int64_t)lead * kChunk) {
      // at most `lead` chunks ahead of the state pass of this head, so that
      // the pass reads the record while the memory-side cache still holds
      // it; a heuristic, so the wait is bounded and then simply ends
      if (tid == 0) {
        const int* f = flags + (slot - lead) * H + h;
        for (int spin = 0; spin < kLeadSpinLimit; ++spin) {
          if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kConsumed) break;
          __builtin_amdgcn_s_sleep(8);
        }
      }
      __syncthreads();
    }
    prep_item<D, SCALAR, RAW, FusedState<VT>::QGB>(q, k, v, log_alpha, beta, H, h, t0, len,
                                                   ws + ((size_t)slot * H + h) * Rec<D>::BYTES, lds, &hdr->status);
    // publish: every wave's record stores acknowledged, then the flag
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (tid == 0) __hip_atomic_store(flags + slot * H + h, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  __shared__ int sTicket;
  int task = blockIdx.x;
  while (task < ntot) {
    int pair, vt;
    task_of<NV>(task, nstate, pair, vt);
    const Sync sy{flags, &hdr->status, lead > 0 && vt == 0 ? flags : nullptr};
    if (pair < N * H)
      state_task<D, VT, FusedState<VT>::NB, FusedState<VT>::HOLD_SF, FusedState<VT>::QGB>(
          cu, H, init, fin, o, ws, sidx, pool_slots, pair / H, pair % H, vt, sy, lds);
    if (tid == 0) sTicket = nstate + atomicAdd(&hdr->state_ticket, 1);
    __syncthreads();
    task = sTicket;
    __syncthreads();
  }
}

// Workspace of the bf16 path: records, then one flag per (slot, head), then
// the header.
static size_t flags_offset(int64_t slots, int H, int d) {
  const size_t rec = d == 128 ? Rec<128>::BYTES : Rec<64>::BYTES;
  return (size_t)slots * H * rec;
}
static size_t hdr_offset(int64_t slots, int H, int d) {
  return flags_offset(slots, H, d) + (((size_t)slots * H * sizeof(int) + 255) & ~(size_t)255);
}

template <int D>
static hipError_t launch_two_kernel(const PrefillArgs& A, int vt, hipStream_t stream) {
  const int64_t slots = prefill_num_slots(A.num_seqs, A.total_tokens);
  const int64_t items = slots * A.num_heads;
  if (A.total_tokens > 0) {
    FusedHdr* hdr = reinterpret_cast<FusedHdr*>((unsigned char*)A.workspace + hdr_offset(slots, A.num_heads, D));
    hipLaunchKernelGGL(fused_init_kernel, dim3(1), dim3(64), 0, stream, (int*)nullptr, (int64_t)0, hdr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    auto kern = A.scalar_gate ? (A.raw_qkb ? prep_kernel<D, true, true> : prep_kernel<D, true, false>)
                              : (A.raw_qkb ? prep_kernel<D, false, true> : prep_kernel<D, false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)items), dim3(kPrepThreads), 0, stream, (const In*)A.q,
                       (const In*)A.k, (const In*)A.v, A.log_alpha, (const In*)A.beta, A.cu_seqlens,
                       A.num_seqs, A.num_heads, (unsigned char*)A.workspace, &hdr->status);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t pairs = (int64_t)A.num_seqs * A.num_heads;
  const int64_t groups = (pairs + 7) / 8;
  const unsigned blocks = (unsigned)(groups * 8 * (D / (16 * vt)));
  auto kern = vt == 4 ? state_kernel<D, 4> : vt == 2 ? state_kernel<D, 2> : state_kernel<D, 1>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), 0, stream, A.cu_seqlens, A.num_seqs, A.num_heads,
                     A.init_state, A.final_state, (In*)A.o, (const unsigned char*)A.workspace, A.state_indices,
                     A.pool_slots);
  return hipGetLastError();
}

// Scheduling overrides for measurements (0: automatic).
#ifndef KDA_PREFILL_SCHEDULE
#define KDA_PREFILL_SCHEDULE 0   // 1: two kernels, 2: one launch
#endif
#ifndef KDA_SLICE_TILES
#define KDA_SLICE_TILES 0
#endif
#ifndef KDA_LEAD_CHUNKS
#define KDA_LEAD_CHUNKS 30   // how far the prep may run ahead of a long pass
#endif

// Returns false (and launches nothing) when the device cannot hold enough
// blocks at once for the one-launch path.
template <int D, int VT>
static bool launch_fused_vt(const PrefillArgs& A, int cus, hipStream_t stream, hipError_t& err) {
  constexpr int NV = D / (16 * VT);
  auto kern = A.scalar_gate ? (A.raw_qkb ? fused_kernel<D, true, true, VT> : fused_kernel<D, true, false, VT>)
                            : (A.raw_qkb ? fused_kernel<D, false, true, VT> : fused_kernel<D, false, false, VT>);
  // state blocks: one per task, at most a quarter of the blocks the device
  // holds at once, in whole groups of 8 NV
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kPrepThreads, 0) != hipSuccess) return false;
  const int cap = ((per_cu * cus / 4) / (8 * NV)) * (8 * NV);
  if (cap < 8 * NV) return false;
  const int64_t pairs = (int64_t)A.num_seqs * A.num_heads;
  const int ntasks = (int)(pairs * NV);
  const int nstate = (int)std::min<int64_t>((((int64_t)ntasks + 8 * NV - 1) / (8 * NV)) * (8 * NV), cap);
  // Sequences that average 64K tokens or more, each pass in a block of its
  // own from the start: the pass is the longer leg, and a prep left to run
  // ahead writes records that are read back from HBM milliseconds later.
  // Keeping it within KDA_LEAD_CHUNKS chunks of the pass lets the pass read
  // them from the memory-side cache instead.  (2^20 tokens, 16 heads, d =
  // 128: 22.0 ms unthrottled; a lead of 16, 24, 28, 30 chunks: 25.4, 19.4,
  // 18.4, 18.2 ms; 32 and more: about 17.7 ms but now and then 23 to 25 ms.
  // The prep's work per chunk is some 20 us, so a short lead starves the
  // pass.)
  const bool throttle = ntasks <= nstate && A.total_tokens >= (int64_t)A.num_seqs * 65536;
  const int lead = throttle ? KDA_LEAD_CHUNKS : 0;

  const int64_t slots = prefill_num_slots(A.num_seqs, A.total_tokens);
  unsigned char* ws = (unsigned char*)A.workspace;
  int* flags = reinterpret_cast<int*>(ws + flags_offset(slots, A.num_heads, D));
  FusedHdr* hdr = reinterpret_cast<FusedHdr*>(ws + hdr_offset(slots, A.num_heads, D));
  const int64_t items = slots * A.num_heads;
  hipLaunchKernelGGL(fused_init_kernel, dim3((unsigned)std::min<int64_t>((items + 255) / 256, 1024)), dim3(256), 0,
                     stream, flags, items, hdr);
  err = hipGetLastError();
  if (err != hipSuccess) return true;
  hipLaunchKernelGGL(kern, dim3((unsigned)(nstate + items)), dim3(kPrepThreads), 0, stream, (const In*)A.q,
                     (const In*)A.k, (const In*)A.v, A.log_alpha, (const In*)A.beta, A.cu_seqlens, A.num_seqs,
                     A.num_heads, A.init_state, A.final_state, (In*)A.o, ws, flags, hdr, A.state_indices,
                     A.pool_slots, nstate, std::max(nstate, ntasks), lead);
  err = hipGetLastError();
  return true;
}

static int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  return cus;
}


template <int D>
static hipError_t launch_t(const PrefillArgs& A, hipStream_t stream) {
  const int cus = device_cus();
  const int64_t pairs = (int64_t)A.num_seqs * A.num_heads;
  if (A.total_tokens == 0 || KDA_PREFILL_SCHEDULE == 1) {
    // Slices of one value tile while they fit the CUs in one round: each
    // chunk step is then shortest.  With more slices than CUs the pass is
    // bound by throughput, and slices of two or four value tiles, which load
    // W, Q' and Kc once for all their columns, do the same work with fewer
    // operand bytes: the widest slice that still gives every CU a workgroup
    // (the results are the same bit for bit).
    const int vt = pairs * (D / 64) >= cus ? 4 : pairs * (D / 32) >= cus ? 2 : 1;
    return launch_two_kernel<D>(A, vt, stream);
  }
  // One launch: value slices of one tile while their tasks are at most a
  // quarter of the blocks (each chunk step is shortest), else two, else four.
  const int vt = KDA_SLICE_TILES ? KDA_SLICE_TILES
                                 : (pairs * (D / 16) <= 2 * cus / 4 ? 1 : pairs * (D / 32) <= 2 * cus / 4 ? 2 : 4);
  hipError_t err = hipSuccess;
  const bool done = vt == 4 ? launch_fused_vt<D, 4>(A, cus, stream, err)
                  : vt == 2 ? launch_fused_vt<D, 2>(A, cus, stream, err)
                            : launch_fused_vt<D, 1>(A, cus, stream, err);
  if (done) return err;
  const int vt2 = pairs * (D / 64) >= cus ? 4 : pairs * (D / 32) >= cus ? 2 : 1;
  return launch_two_kernel<D>(A, vt2, stream);
}

}  // namespace bf

size_t prefill_record_bytes_bf16(int d) { return d == 128 ? bf::Rec<128>::BYTES : bf::Rec<64>::BYTES; }

size_t prefill_workspace_bytes_bf16(int64_t slots, int num_heads, int d) {
  return bf::hdr_offset(slots, num_heads, d) + sizeof(bf::FusedHdr);
}

size_t prefill_status_offset_bf16(int64_t slots, int num_heads, int d) {
  return bf::hdr_offset(slots, num_heads, d) + offsetof(bf::FusedHdr, status);
}

hipError_t clear_prefill_status(int* status, hipStream_t stream) {
  hipLaunchKernelGGL(bf::clear_status_kernel, dim3(1), dim3(64), 0, stream, status);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs& A, hipStream_t stream) {
  if (A.num_seqs == 0) return hipSuccess;
  return A.d == 128 ? bf::launch_t<128>(A, stream) : bf::launch_t<64>(A, stream);
}

}  // namespace kda
