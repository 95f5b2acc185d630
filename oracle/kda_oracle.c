/*
 * kda_oracle.c -- plain fp64 CPU oracle of the Kimi Delta Attention (KDA)
 * recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The GPU library never links,
 * calls or includes anything from here, and nothing here comes from it.
 *
 * What it computes (page "Kimi Delta Attention", architecture deep dive,
 * §03 "KDA's specific innovation", the recurrence attributed to Moonshot):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *
 * with the read-out of §02 ("From additive memory to corrective memory"):
 *
 *     o_t = S_t^T q_t            (after the update of token t)
 *
 * S is dk x dv (rows = key channels i, columns = value channels j).  Read
 * right to left, as §03 says: first every key channel (row of S) decays by
 * its own alpha_t[i]; then the delta-rule erase along k_t acts on that
 * decayed state; then the new association k_t v_t^T is written.  Expanding
 * the product gives the rank-1 form this file executes token by token:
 *
 *     D    = Diag(alpha_t) S_{t-1}                       (decay)
 *     p    = D^T k_t                                     (read at the key)
 *     e    = beta_t (v_t - p)                            (scaled error)
 *     S_t  = D + k_t e^T                                 (correct / write)
 *     o_t  = S_t^T q_t
 *
 * since (I - b k k^T) D + b k v^T = D + b k (v - D^T k)^T.
 *
 * alpha_t = exp(log_alpha_t) is evaluated here in fp64 (the input is the
 * natural log of the channel gate, alpha in (0,1) as the "Kimi Linear Guide"
 * page's "Channel-Wise Data-Dependent Gating" section gives it).
 *
 * Storage: the state of one (sequence, head) is kept as S^T, i.e.
 * state[j][i] = S_{ij} with the key index i contiguous.  Inputs are cast
 * exactly to fp64 (bf16 and fp32 both embed exactly in binary64).
 *
 * Test-only switch: mode = KDA_ORACLE_ERASE_OFF replaces the error by
 * e = beta_t v_t, i.e. the plain additive write of §02's linear attention
 * with the same channel decay.  It exists so that the decay and write parts
 * can be checked against closed forms with the erase taken out.
 *
 * Work is split over (sequence, head, block of value channels) units.  Value
 * columns of S never mix in the recurrence, so the split changes no
 * arithmetic: every output element is produced by the same sequence of fp64
 * operations whatever the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { KDA_ORACLE_F32 = 0, KDA_ORACLE_BF16 = 1, KDA_ORACLE_F64 = 2 };
enum { KDA_ORACLE_KDA = 0, KDA_ORACLE_ERASE_OFF = 1 };
enum { VBLOCK = 16 };

/* One element of a typed input array as fp64 (exact for all three types). */
static double load_elem(const void* base, int type, int64_t idx) {
  if (type == KDA_ORACLE_F64) return ((const double*)base)[idx];
  if (type == KDA_ORACLE_F32) return (double)((const float*)base)[idx];
  /* bf16: the upper 16 bits of an IEEE binary32 */
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

typedef struct {
  const void *q, *k, *v, *log_alpha, *beta;
  int in_type, la_type;
  const int64_t* cu_seqlens;
  int num_seqs;
  const double* init_state;
  double* o;
  const int64_t* out_rows;
  int64_t n_out_rows;
  double* final_state;
  int H, dk, dv;
  int mode;
  int64_t n_units;
  int64_t next_unit; /* shared work counter */
} job_t;

/* First index in the sorted out_rows list that is >= t. */
static int64_t lower_bound_rows(const int64_t* rows, int64_t n, int64_t t) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (rows[mid] < t) lo = mid + 1; else hi = mid;
  }
  return lo;
}

/* Token loop of one (sequence n, head h, value columns [j0, j0+w)). */
static void run_unit(const job_t* J, int64_t u, double* S, double* a,
                     double* kk, double* qq) {
  const int H = J->H, dk = J->dk, dv = J->dv;
  const int nvb = (dv + VBLOCK - 1) / VBLOCK;
  const int vb = (int)(u % nvb);
  const int h = (int)((u / nvb) % H);
  const int n = (int)(u / ((int64_t)nvb * H));
  const int j0 = vb * VBLOCK;
  const int w = (dv - j0) < VBLOCK ? (dv - j0) : VBLOCK;
  const int64_t bos = J->cu_seqlens[n], eos = J->cu_seqlens[n + 1];
  const int64_t sbase = ((int64_t)n * H + h) * dv * dk; /* state[n][h] */

  /* S[jj][i] = S_{i, j0+jj}: the block's columns, key index contiguous */
  for (int jj = 0; jj < w; ++jj)
    for (int i = 0; i < dk; ++i)
      S[jj * dk + i] = J->init_state ? J->init_state[sbase + (int64_t)(j0 + jj) * dk + i] : 0.0;

  int64_t r = J->out_rows ? lower_bound_rows(J->out_rows, J->n_out_rows, bos) : 0;

  for (int64_t t = bos; t < eos; ++t) {
    const int64_t kb = (t * H + h) * dk; /* [T,H,dk] */
    const int64_t vbase = (t * H + h) * dv; /* [T,H,dv] */
    for (int i = 0; i < dk; ++i) {
      a[i] = exp(load_elem(J->log_alpha, J->la_type, kb + i));
      kk[i] = load_elem(J->k, J->in_type, kb + i);
      qq[i] = load_elem(J->q, J->in_type, kb + i);
    }
    const double beta = load_elem(J->beta, J->in_type, t * H + h);

    for (int jj = 0; jj < w; ++jj) {
      double* Sj = S + jj * dk; /* column j0+jj of S */
      /* decay: row i of S (key channel i) scales by alpha_t[i] */
      for (int i = 0; i < dk; ++i) Sj[i] *= a[i];
      /* read the decayed state at the key: p_j = sum_i S_ij k_i */
      double p = 0.0;
      for (int i = 0; i < dk; ++i) p += Sj[i] * kk[i];
      /* scaled error (or the plain additive write with the erase off) */
      const double vj = load_elem(J->v, J->in_type, vbase + j0 + jj);
      const double e = (J->mode == KDA_ORACLE_ERASE_OFF) ? beta * vj : beta * (vj - p);
      /* write: S += k e^T */
      for (int i = 0; i < dk; ++i) Sj[i] += kk[i] * e;
      /* read-out after the update: o_j = sum_i S_ij q_i */
      double oj = 0.0;
      for (int i = 0; i < dk; ++i) oj += Sj[i] * qq[i];

      int64_t orow = -1;
      if (!J->out_rows) orow = t;
      else if (r < J->n_out_rows && J->out_rows[r] == t) orow = r;
      if (orow >= 0 && J->o) J->o[(orow * H + h) * dv + j0 + jj] = oj;
    }
    if (J->out_rows && r < J->n_out_rows && J->out_rows[r] == t) ++r;
  }

  if (J->final_state)
    for (int jj = 0; jj < w; ++jj)
      for (int i = 0; i < dk; ++i)
        J->final_state[sbase + (int64_t)(j0 + jj) * dk + i] = S[jj * dk + i];
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int dk = J->dk;
  double* S = (double*)malloc(sizeof(double) * (size_t)VBLOCK * dk);
  double* a = (double*)malloc(sizeof(double) * (size_t)dk * 3);
  if (!S || !a) { free(S); free(a); return (void*)1; }
  for (;;) {
    int64_t u = __atomic_fetch_add(&J->next_unit, 1, __ATOMIC_RELAXED);
    if (u >= J->n_units) break;
    run_unit(J, u, S, a, a + dk, a + 2 * dk);
  }
  free(S);
  free(a);
  return NULL;
}

/*
 * Variable-length prefill over packed sequences.
 *   q, k       : [T, H, dk]   in in_type
 *   v          : [T, H, dv]   in in_type
 *   log_alpha  : [T, H, dk]   in la_type (F32 or F64), natural log of alpha
 *   beta       : [T, H]       in in_type
 *   cu_seqlens : host int64 [num_seqs + 1], cu[0] = 0, non-decreasing
 *   init_state : fp64 [num_seqs, H, dv, dk] or NULL (zero state)
 *   o          : fp64 [T, H, dv], or [n_out_rows, H, dv] when out_rows is given
 *   out_rows   : NULL, or a sorted list of token indices whose outputs are kept
 *   final_state: fp64 [num_seqs, H, dv, dk] or NULL; may alias init_state
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
int kda_oracle_prefill(const void* q, const void* k, const void* v,
                       const void* log_alpha, const void* beta,
                       int in_type, int la_type,
                       const int64_t* cu_seqlens, int num_seqs,
                       const double* init_state, double* o,
                       const int64_t* out_rows, int64_t n_out_rows,
                       double* final_state,
                       int H, int dk, int dv, int mode, int nthreads) {
  if (!q || !k || !v || !log_alpha || !beta || !cu_seqlens) return -1;
  if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (in_type < 0 || in_type > 2 || (la_type != KDA_ORACLE_F32 && la_type != KDA_ORACLE_F64)) return -1;
  if (mode != KDA_ORACLE_KDA && mode != KDA_ORACLE_ERASE_OFF) return -1;
  if (nthreads < 1) nthreads = 1;

  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta;
  J.in_type = in_type; J.la_type = la_type;
  J.cu_seqlens = cu_seqlens; J.num_seqs = num_seqs;
  J.init_state = init_state; J.o = o;
  J.out_rows = out_rows; J.n_out_rows = n_out_rows;
  J.final_state = final_state;
  J.H = H; J.dk = dk; J.dv = dv; J.mode = mode;
  J.n_units = (int64_t)num_seqs * H * ((dv + VBLOCK - 1) / VBLOCK);
  J.next_unit = 0;

  if (nthreads > J.n_units) nthreads = (int)(J.n_units > 0 ? J.n_units : 1);
  if (nthreads == 1) return worker(&J) ? -2 : 0;

  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -2;
  int started = 0, rc = 0;
  for (; started < nthreads; ++started)
    if (pthread_create(&th[started], NULL, worker, &J) != 0) break;
  if (started == 0) rc = worker(&J) ? -2 : 0;
  for (int i = 0; i < started; ++i) {
    void* ret = NULL;
    pthread_join(th[i], &ret);
    if (ret) rc = -2;
  }
  free(th);
  return rc;
}
