// kda_prefill.hip -- chunk-parallel KDA prefill over packed varlen sequences,
// fp32 inputs (the bf16 path is kda_prefill_bf16.hip; both share the chunk
// equations and the slot map below).
//
// The recurrence (page "Kimi Delta Attention", §03)
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t
// is evaluated in chunks of C = 64 tokens (§06 "chunk-parallel KDA": matrix
// products inside a block, only the final state crosses block boundaries;
// the "Kimi Linear Guide" page's hardware-chunking section uses B = 64).
// The pages give the outline only; the chunk equations below follow from the
// recurrence by unrolling it over one chunk.  For a chunk with tokens
// r = 0..C-1 (a partial chunk is padded with k = q = v = 0, beta = 0,
// log_alpha = 0, which leaves every result unchanged) and entering state S0:
//
//   G[r,i]  = sum_{s<=r} log_alpha[s,i]          cumulative log decay (fp32)
//   Kg = K * e^G      Qg = Q * e^G      Kc = K * e^(G[C-1] - G)
//   A[r,j]  = sum_i k_r[i] k_j[i] e^(G[r,i]-G[j,i])   for j < r, else 0
//   Bqk[r,j]= sum_i q_r[i] k_j[i] e^(G[r,i]-G[j,i])   for j <= r, else 0
//   T       = (I + Diag(beta) A)^-1      (unit lower triangular)
//   W = T Diag(beta) Kg          U = T Diag(beta) V
//   E       = U - W S0           row r = beta_r (v_r - (Diag(a_r) S_{r-1})^T k_r)
//   O       = Qg S0 + Bqk E
//   S_end   = Diag(e^G[C-1]) S0 + Kc^T E
//
// The decays e^(G[r]-G[j]) inside A and Bqk are formed as a product of two
// factors anchored at token m = 31, X = e^(G - G[m]) and 1/X, so that no
// factor leaves the fp32 range for |log_alpha| <= 2.5 (the numerical-range
// concern of §08 item 3).
//
// Kernel 1 (prep, one workgroup per chunk and head, all chunks in parallel)
// computes G, A, Bqk, T, W, U, Qg, Kc and writes them to the workspace as
// MFMA operand fragments (see kda_device.h for the fragment map).
// Kernel 2 (state pass, one workgroup per (sequence, head, 16 value
// columns)) walks the chunks of its sequence in order with its 128 x 16
// slice of S resident in accumulator registers: value columns of S never mix
// in the recurrence, so the slices are independent.
#include "kda_device.h"
#include "kda_launch.h"
#include "kda_prefill_common.h"

namespace kda {

// ---------------------------------------------------------------------------
// Per (chunk slot, head) record in the workspace: the state pass's operands
// as fp32 MFMA fragments.
// ---------------------------------------------------------------------------
template <int D>
struct Rec {
  static constexpr int KB = D / 32;                 // 32-deep key blocks
  static constexpr int NT = D / 16;                 // 16-wide key / value tiles
  static constexpr size_t FB = 64 * 8 * 4;          // bytes per fragment
  static constexpr size_t W = 0;                       // [4 token tiles][KB]       W    (row token, k key)
  static constexpr size_t Q = W + 4 * KB * FB;         // [4][KB]                   Qg   (row token, k key)
  static constexpr size_t KC = Q + 4 * KB * FB;        // [NT key tiles][2]         Kc^T (row key, k token)
  static constexpr size_t B = KC + NT * 2 * FB;        // [4 token tiles][2]        Bqk  (row token, k token)
  static constexpr size_t U = B + 8 * FB;              // [NT value tiles][4 token tiles][64] f32x4
  static constexpr size_t G = U + (size_t)NT * 4 * 64 * 16;  // [D] fp32 e^G[C-1]
  static constexpr size_t BYTES = G + (size_t)D * 4;
};

using Frag = f32x8;
using Half = f32x4;

__device__ __forceinline__ Frag frag8(const float (&v)[8]) {
  Frag f;
#pragma unroll
  for (int m = 0; m < 8; ++m) f[m] = v[m];
  return f;
}

// Chunk slots: chunk c of sequence n lives in slot cu[n]/64 + n + c.  Slots
// of different sequences never collide (floor(a/64) + ceil(L/64) <=
// floor((a+L)/64) + 1), and every slot is below T/64 + N + 1.
int64_t prefill_num_slots(int32_t num_seqs, int64_t total_tokens) {
  return total_tokens / kChunk + num_seqs + 1;
}

size_t prefill_record_bytes_f32(int d) { return d == 128 ? Rec<128>::BYTES : Rec<64>::BYTES; }

// The status word follows the records.
size_t prefill_status_offset_f32(int64_t slots, int num_heads, int d) {
  return (size_t)slots * num_heads * prefill_record_bytes_f32(d);
}

// ---------------------------------------------------------------------------
// Kernel 1: per-chunk factors.  512 threads (8 waves) per (chunk, head).
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 512;

template <int D>
__global__ __launch_bounds__(kPrepThreads) void prefill_prep_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta, const int32_t* __restrict__ cu, int N,
    int H, unsigned char* __restrict__ ws, int scalar_gate, int raw_qkb, int* __restrict__ status) {
  using In = float;
  using R = Rec<D>;
  constexpr int C = kChunk;
  constexpr int NTH = kPrepThreads;
  constexpr int NW = NTH / 64;                       // waves
  constexpr int PI = D + 16 / (int)sizeof(In);       // row pitch of staged inputs (+16 bytes)
  constexpr int PX = D + 4;                          // row pitch of X
  constexpr int PL = C + 4;                          // row pitch of L and T
  constexpr int KB = D / 32, NT = D / 16;
  constexpr size_t FS = sizeof(Frag);
  constexpr int QBYTES = (C * PI * (int)sizeof(In)) > (C * PL * 4) ? (C * PI * (int)sizeof(In)) : (C * PL * 4);

  __shared__ __align__(16) In sK[C][PI];
  __shared__ __align__(16) unsigned char sQraw[QBYTES];   // Q, later T
  __shared__ __align__(16) float sX[C][PX];               // X = e^(G - G[m])
  __shared__ __align__(16) float sL[C][PL];               // Diag(beta) A (strictly lower)
  __shared__ float sEgm[D], sEcm[D], sGm[D], sGc[D], sBeta[C];
  __shared__ float sSeg[NTH / 64][D];
  __shared__ float sNrm[2][C];                            // raw inputs: 1/|k|, 1/|q| per token
  __shared__ float sScr[4][16][17];
  In (*sQ)[PI] = reinterpret_cast<In (*)[PI]>(sQraw);
  float (*sT)[PL] = reinterpret_cast<float (*)[PL]>(sQraw);

  const int64_t slot = blockIdx.x;
  const int h = blockIdx.y;
  int n, len;
  int64_t t0;
  if (!decode_slot(cu, N, slot, n, t0, len)) return;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 4, l16 = l & 15;
  unsigned char* rec = ws + ((size_t)slot * H + h) * R::BYTES;

  // ---- phase 1: stage K and Q rows, beta; clear L -------------------------
  {
    constexpr int EV = 16 / (int)sizeof(In);  // elements per 16-byte vector
    constexpr int VR = D / EV;                // vectors per row
    for (int idx = tid; idx < C * VR; idx += NTH) {
      const int r = idx / VR, cv = idx % VR;
      uint4 kq = {0, 0, 0, 0}, qq = {0, 0, 0, 0};
      if (r < len) {
        const int64_t off = ((t0 + r) * H + h) * D + cv * EV;
        kq = *reinterpret_cast<const uint4*>(k + off);
        qq = *reinterpret_cast<const uint4*>(q + off);
      }
      *reinterpret_cast<uint4*>(&sK[r][cv * EV]) = kq;
      *reinterpret_cast<uint4*>(&sQ[r][cv * EV]) = qq;
    }
    if (tid < C) {
      const float b = tid < len ? beta[(t0 + tid) * H + h] : 0.f;
      sBeta[tid] = (raw_qkb && tid < len) ? sigmoid(b) : b;
    }
    for (int idx = tid; idx < C * PL; idx += NTH) (&sL[0][0])[idx] = 0.f;
  }
  if (raw_qkb) {   // unit q and k rows, in place
    __syncthreads();
    if (tid < 2 * C) {
      const int r = tid % C;
      const In* row = tid < C ? &sK[r][0] : &sQ[r][0];
      float ss = 0.f;
      for (int i = 0; i < D; ++i) ss += row[i] * row[i];
      sNrm[tid / C][r] = inv_norm(ss);
    }
    __syncthreads();
    for (int idx = tid; idx < C * D; idx += NTH) {
      const int r = idx / D, i = idx % D;
      sK[r][i] *= sNrm[0][r];
      sQ[r][i] *= sNrm[1][r];
    }
    __syncthreads();
  }

  // ---- phase 2: cumulative log decay and the anchored factor X -------------
  {
    constexpr int SEGS = NTH / D;        // token segments per channel
    constexpr int SL = C / SEGS;         // tokens per segment
    const int i = tid % D, s = tid / D;
    float gl[SL];
    float run = 0.f;
#pragma unroll
    for (int r = 0; r < SL; ++r) {
      const int tok = s * SL + r;
      const int64_t th = (t0 + tok) * H + h;
      const float x = tok < len ? log_alpha[scalar_gate ? th : th * D + i] : 0.f;
      run += x;
      gl[r] = run;
    }
    sSeg[s][i] = run;
    __syncthreads();
    float off = 0.f;
    for (int s2 = 0; s2 < s; ++s2) off += sSeg[s2][i];
#pragma unroll
    for (int r = 0; r < SL; ++r) gl[r] += off;
    constexpr int M = 31;
    if (s == M / SL) sGm[i] = gl[M % SL];
    if (s == SEGS - 1) sGc[i] = gl[SL - 1];
    __syncthreads();
    const float gm = sGm[i], gc = sGc[i];
    float dgmax = 0.f;
#pragma unroll
    for (int r = 0; r < SL; ++r) {
      sX[s * SL + r][i] = __expf(gl[r] - gm);
      dgmax = fmaxf(dgmax, fabsf(gl[r] - gm));
    }
    // a gate sum beyond the fp32 exponent range: report it (results of this
    // chunk may be non-finite)
    if (__any(dgmax > kMaxAnchoredExp) && l == 0)
      __hip_atomic_fetch_or(status, kStatusGateRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (s == 0) {
      sEgm[i] = __expf(gm);
      sEcm[i] = __expf(gc - gm);
      reinterpret_cast<float*>(rec + R::G)[i] = __expf(gc);
    }
  }
  __syncthreads();

  // ---- phase 3: A and Bqk^T tiles (MFMA), Qg fragments ----------------------
  {
    // fragment of a token-major operand: row `row`, key block p, times X or 1/X
    auto row_frag = [&](const In (*src)[PI], int row, int p, bool inv, float (&vals)[8]) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int key = 32 * p + 16 * hh + 4 * g;
        const f32x4 a = lds4(&src[row][key]);
        const f32x4 x = *reinterpret_cast<const f32x4*>(&sX[row][key]);
#pragma unroll
        for (int e = 0; e < 4; ++e) vals[4 * hh + e] = inv ? a[e] * __builtin_amdgcn_rcpf(x[e]) : a[e] * x[e];
      }
    };
    for (int pi = w; pi < 10; pi += NW) {
      // lower-triangular tile pairs (rt, jt), jt <= rt, in row order
      const int rt = pi < 1 ? 0 : pi < 3 ? 1 : pi < 6 ? 2 : 3;
      const int jt = pi - (rt * (rt + 1)) / 2;
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        float va[8], vb[8], vq[8];
        row_frag(sK, 16 * rt + l16, p, false, va);   // Ka: k_r e^(G_r - G_m)
        row_frag(sK, 16 * jt + l16, p, true, vb);    // Kbar: k_j e^(G_m - G_j)
        row_frag(sQ, 16 * rt + l16, p, false, vq);   // Qa: q_r e^(G_r - G_m)
        const Frag ka = frag8(va), kb = frag8(vb), qa = frag8(vq);
        mma(accA, ka, kb);   // A[r][j]
        mma(accB, kb, qa);   // Bqk^T[j][r]
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rt + 4 * g + e, j = 16 * jt + l16;
        sL[r][j] = (j < r) ? sBeta[r] * accA[e] : 0.f;
      }
      // Bqk fragment (row tile rt, token block jt/2): lane l holds row
      // r = 16 rt + l16 and columns j = 16 jt + 4 g + e
      Half hb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * jt + 4 * g + e, r = 16 * rt + l16;
        hb[e] = j <= r ? accB[e] : 0.f;
      }
      const size_t foff = ((size_t)(rt * 2 + jt / 2) * 64 + l) * FS + 4 * (jt & 1) * sizeof(In);
      *reinterpret_cast<Half*>(rec + R::B + foff) = hb;
      if (jt == rt && (rt & 1) == 0) {   // columns above the diagonal block
        const size_t zoff = ((size_t)(rt * 2 + jt / 2) * 64 + l) * FS + 4 * sizeof(In);
        *reinterpret_cast<Half*>(rec + R::B + zoff) = Half{0.f, 0.f, 0.f, 0.f};
      }
    }
    // Qg fragments (token tile rt, key block p)
    for (int f = w; f < 4 * KB; f += NW) {
      const int rt = f / KB, p = f % KB;
      float vq[8];
      row_frag(sQ, 16 * rt + l16, p, false, vq);
#pragma unroll
      for (int m = 0; m < 8; ++m) vq[m] *= sEgm[32 * p + kpos(g, m)];
      *reinterpret_cast<Frag*>(rec + R::Q + ((size_t)f * 64 + l) * FS) = frag8(vq);
    }
  }
  __syncthreads();   // Q is dead from here on: its space becomes T

  // ---- phase 4: T = (I + L)^-1, L = Diag(beta) A strictly lower ------------
  // 16 x 16 diagonal blocks by forward substitution, then block doubling:
  //   [[X, 0], [Y, Z]]^-1 = [[X^-1, 0], [-Z^-1 Y X^-1, Z^-1]]
  // first for the 16-blocks (1,0) and (3,2), then for the 32-block (1,0).
  {
    for (int idx = tid; idx < C * PL; idx += NTH) (&sT[0][0])[idx] = 0.f;
    __syncthreads();
    if (w == 0) {
      const int bk = l >> 4, c = l & 15;   // lane = (block, column)
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < r; ++j) acc -= sL[16 * bk + r][16 * bk + j] * x[j];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[16 * bk + r][16 * bk + c] = x[r];
    }
    __syncthreads();
    const int c = l16, r0 = 4 * g;
    // 16-block doubling: wave 0 -> block (1,0), wave 1 -> block (3,2)
    if (w < 2) {
      const int a = 2 * w, bb = a + 1;
      float x[4] = {0.f, 0.f, 0.f, 0.f};
      for (int qq = 0; qq < 16; ++qq) {
        const float tv = sT[16 * a + qq][16 * a + c];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] += sL[16 * bb + r0 + e][16 * a + qq] * tv;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sScr[w][r0 + e][c] = x[e];
    }
    __syncthreads();
    if (w < 2) {
      const int a = 2 * w, bb = a + 1;
      float y[4] = {0.f, 0.f, 0.f, 0.f};
      for (int qq = 0; qq < 16; ++qq) {
        const float tv = sScr[w][qq][c];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] -= sT[16 * bb + r0 + e][16 * bb + qq] * tv;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[16 * bb + r0 + e][16 * a + c] = y[e];
    }
    __syncthreads();
    // 32-block doubling: Y = L[32:64, 0:32] T[0:32, 0:32], then
    // T[32:64, 0:32] = -T[32:64, 32:64] Y; wave w < 4 owns 16-tile (bi, bj)
    if (w < 4) {
      const int bi = w >> 1, bj = w & 1;
      float y[4] = {0.f, 0.f, 0.f, 0.f};
      for (int kb = bj; kb < 2; ++kb)
        for (int qq = 0; qq < 16; ++qq) {
          const float tv = sT[16 * kb + qq][16 * bj + c];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] += sL[32 + 16 * bi + r0 + e][16 * kb + qq] * tv;
        }
#pragma unroll
      for (int e = 0; e < 4; ++e) sScr[w][r0 + e][c] = y[e];
    }
    __syncthreads();
    if (w < 4) {
      const int bi = w >> 1, bj = w & 1;
      float z[4] = {0.f, 0.f, 0.f, 0.f};
      for (int kb = 0; kb <= bi; ++kb)
        for (int qq = 0; qq < 16; ++qq) {
          const float tv = sScr[2 * kb + bj][qq][c];
#pragma unroll
          for (int e = 0; e < 4; ++e) z[e] -= sT[32 + 16 * bi + r0 + e][32 + 16 * kb + qq] * tv;
        }
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[32 + 16 * bi + r0 + e][16 * bj + c] = z[e];
    }
    __syncthreads();
  }

  // ---- phase 5: W^T = Kg^T T'^T and U = T' V with T' = T Diag(beta);
  //               Kc^T fragments ---------------------------------------------
  {
    // T' fragments (row tile rt, token block p): the B operand of W^T and
    // the A operand of U (the two layouts coincide)
    Frag tf[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float vals[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int j = 32 * p + kpos(g, m);
          vals[m] = sT[16 * rt + l16][j] * sBeta[j];
        }
        tf[rt][p] = frag8(vals);
      }
    // tasks 0..NT-1: key tile (W, Kc); NT..2NT-1: value tile (U)
    for (int task = w; task < 2 * NT; task += NW) {
      if (task < NT) {
        const int it = task;
        const int col = 16 * it + l16;   // key channel of this lane
        Frag kg[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float vg[8], vc[8];
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const int j = 32 * p + kpos(g, m);
            const float kx = sK[j][col];
            const float x = sX[j][col];
            vg[m] = kx * x * sEgm[col];
            vc[m] = kx * __builtin_amdgcn_rcpf(x) * sEcm[col];
          }
          kg[p] = frag8(vg);
          *reinterpret_cast<Frag*>(rec + R::KC + ((size_t)(it * 2 + p) * 64 + l) * FS) = frag8(vc);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          f32x4 accW = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (p > (rt >> 1)) break;   // T'[r][j] = 0 for j > r
            mma(accW, kg[p], tf[rt][p]);
          }
          const size_t off = ((size_t)(rt * KB + it / 2) * 64 + l) * FS + 4 * (it & 1) * sizeof(In);
          *reinterpret_cast<Half*>(rec + R::W + off) = accW;
        }
      } else {
        const int ct = task - NT;
        const int col = 16 * ct + l16;   // value channel of this lane
        Frag vf[2];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const int j = 32 * p + kpos(g, m);
            vf[p][m] = j < len ? v[((t0 + j) * H + h) * D + col] : 0.f;
          }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          f32x4 accU = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            if (p > (rt >> 1)) break;
            mma(accU, tf[rt][p], vf[p]);
          }
          *reinterpret_cast<f32x4*>(rec + R::U + ((size_t)(ct * 4 + rt) * 64 + l) * 16) = accU;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: sequential pass over the chunks of one (sequence, head) for a
// 16-column slice of S.  Wave w owns key rows [D/4 w, D/4 (w+1)) of the
// slice as accumulators and token tile w of every chunk.  The operands of
// chunk c+1 are loaded into registers while chunk c is computed.
// ---------------------------------------------------------------------------
template <int D>
struct ChunkOps {
  static constexpr int KB = D / 32, KTW = D / 64;
  Frag w[KB];          // W, token tile of this wave
  Frag q[KB];          // Qg
  Frag kc[KTW][2];     // Kc^T, key tiles of this wave
  Frag b[2];           // Bqk
  f32x4 u;             // U, token tile of this wave, this value slice
  f32x4 gam[KTW];      // e^G[C-1] for this lane's key rows
};

template <int D>
__device__ __forceinline__ void load_ops(ChunkOps<D>& o, const unsigned char* __restrict__ rec, int w, int l, int g,
                                         int vt) {
  using R = Rec<D>;
  using O = ChunkOps<D>;
  constexpr size_t FS = sizeof(Frag);
#pragma unroll
  for (int p = 0; p < O::KB; ++p)
    o.w[p] = *reinterpret_cast<const Frag*>(rec + R::W + ((size_t)(w * O::KB + p) * 64 + l) * FS);
#pragma unroll
  for (int p = 0; p < O::KB; ++p)
    o.q[p] = *reinterpret_cast<const Frag*>(rec + R::Q + ((size_t)(w * O::KB + p) * 64 + l) * FS);
#pragma unroll
  for (int kt = 0; kt < O::KTW; ++kt)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int kti = w * O::KTW + kt;
      o.kc[kt][p] = *reinterpret_cast<const Frag*>(rec + R::KC + ((size_t)(kti * 2 + p) * 64 + l) * FS);
    }
  // both token blocks of Bqk are loaded (the second is unused for w < 2) so
  // that every chunk issues the same loads and the waits stay exact
#pragma unroll
  for (int p = 0; p < 2; ++p)
    o.b[p] = *reinterpret_cast<const Frag*>(rec + R::B + ((size_t)(w * 2 + p) * 64 + l) * FS);
  o.u = *reinterpret_cast<const f32x4*>(rec + R::U + ((size_t)(vt * 4 + w) * 64 + l) * 16);
#pragma unroll
  for (int kt = 0; kt < O::KTW; ++kt)
    o.gam[kt] = *reinterpret_cast<const f32x4*>(rec + R::G + (size_t)(16 * (w * O::KTW + kt) + 4 * g) * 4);
}

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_state_kernel(
    const int32_t* __restrict__ cu, int N, int H, const float* init, float* fin, float* __restrict__ o,
    const unsigned char* __restrict__ ws, const int32_t* __restrict__ sidx, int pool_slots) {
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

  __shared__ Frag sS[KB][64];   // S as the B operand
  __shared__ Frag sE[2][64];    // E as the B operand

  const int64_t sslot = state_slot(sidx, pool_slots, n);
  if (sslot < 0) init = nullptr, fin = nullptr;
  const int64_t sbase = (sslot * H + h) * D;   // row (value channel) base of state[slot][h]
  f32x4 S[KTW];
#pragma unroll
  for (int kt = 0; kt < KTW; ++kt) {
    const int kti = w * KTW + kt;
    S[kt] = init ? *reinterpret_cast<const f32x4*>(init + (sbase + col) * D + 16 * kti + 4 * g)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto rec_of = [&](int c) { return ws + ((size_t)(slot0 + min(c, nch - 1)) * H + h) * R::BYTES; };

  // one chunk step with operands `ops`
  auto step = [&](const ChunkOps<D>& ops, int c) {
    const int64_t t0 = bos + (int64_t)c * kChunk;
    const int len = (int)min<int64_t>(kChunk, eos - t0);

    // S as the B operand (reduction over keys)
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      const int kti = w * KTW + kt;
      *reinterpret_cast<Half*>(reinterpret_cast<float*>(&sS[kti >> 1][l]) + 4 * (kti & 1)) = S[kt];
    }
    __syncthreads();

    // token tile w: W S0 and Qg S0
    f32x4 wsum = {0.f, 0.f, 0.f, 0.f}, qsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KB; ++p) {
      const Frag sh = sS[p][l];
      mma(wsum, ops.w[p], sh);
      mma(qsum, ops.q[p], sh);
    }
    // E = U - W S0 for token tile w, published as the B operand of the
    // reductions over tokens
    *reinterpret_cast<Half*>(reinterpret_cast<float*>(&sE[w >> 1][l]) + 4 * (w & 1)) = ops.u - wsum;
    __syncthreads();

    // S <- Diag(e^G[C-1]) S + Kc^T E  (this wave's key tiles)
#pragma unroll
    for (int kt = 0; kt < KTW; ++kt) {
      S[kt] *= ops.gam[kt];
#pragma unroll
      for (int p = 0; p < 2; ++p) mma(S[kt], ops.kc[kt][p], sE[p][l]);
    }
    // O = Qg S0 + Bqk E for token tile w (token blocks p <= w/2)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (p > (w >> 1)) break;
      mma(qsum, ops.b[p], sE[p][l]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * w + 4 * g + e;
      if (r < len) o[((t0 + r) * H + h) * D + col] = qsum[e];
    }
  };

  // ping-pong buffers: the loads for chunk c+1 are in flight while chunk c
  // is computed; every iteration issues the same loads (past the last
  // chunk the last record is read again), so the compiler's waits stay exact
  ChunkOps<D> bufA, bufB;
  if (nch > 0) load_ops<D>(bufA, rec_of(0), w, l, g, vt);
  for (int c = 0; c < nch; c += 2) {
    load_ops<D>(bufB, rec_of(c + 1), w, l, g, vt);
    step(bufA, c);
    if (c + 1 >= nch) break;
    load_ops<D>(bufA, rec_of(c + 2), w, l, g, vt);
    step(bufB, c + 1);
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
static hipError_t launch_prefill_t(const PrefillArgs& A, hipStream_t stream) {
  const int64_t slots = prefill_num_slots(A.num_seqs, A.total_tokens);
  if (A.total_tokens > 0) {
    int* status = reinterpret_cast<int*>((unsigned char*)A.workspace + prefill_status_offset_f32(slots, A.num_heads, D));
    hipError_t e = clear_prefill_status(status, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_prep_kernel<D>), dim3((unsigned)slots, (unsigned)A.num_heads), dim3(kPrepThreads), 0,
                       stream, (const float*)A.q, (const float*)A.k, (const float*)A.v, A.log_alpha,
                       (const float*)A.beta, A.cu_seqlens, A.num_seqs, A.num_heads, (unsigned char*)A.workspace,
                       (int)A.scalar_gate, (int)A.raw_qkb, status);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t pairs = (int64_t)A.num_seqs * A.num_heads;
  const int64_t groups = (pairs + 7) / 8;
  const unsigned blocks = (unsigned)(groups * 8 * (D / 16));
  hipLaunchKernelGGL((prefill_state_kernel<D>), dim3(blocks), dim3(kThreads), 0, stream, A.cu_seqlens, A.num_seqs,
                     A.num_heads, A.init_state, A.final_state, (float*)A.o, (const unsigned char*)A.workspace,
                     A.state_indices, A.pool_slots);
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& A, hipStream_t stream) {
  if (A.num_seqs == 0) return hipSuccess;
  return A.d == 128 ? launch_prefill_t<128>(A, stream) : launch_prefill_t<64>(A, stream);
}

}  // namespace kda
