/*
 * kda_oracle_grad.c -- plain fp64 CPU oracle of the gradients of the Kimi
 * Delta Attention recurrence (reverse mode, token by token).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The GPU library never links,
 * calls or includes anything from here, and nothing here comes from it.
 *
 * The forward map is the recurrence of the page "Kimi Delta Attention"
 * (§03 "KDA's specific innovation") with the read-out of §02, executed in its
 * rank-1 form exactly as kda_oracle.c does:
 *
 *     D   = Diag(alpha_t) S_{t-1}          alpha_t = exp(log_alpha_t)
 *     p   = D^T k_t
 *     e   = beta_t (v_t - p)
 *     S_t = D + k_t e^T
 *     o_t = S_t^T q_t
 *
 * §06 of that page names training as the other user of the chunkwise form;
 * the pages write no gradient out, so this file states it: for a scalar loss
 * L with dL/do_t = do_t and dL/dS_T = dS_T, walk the tokens backwards with
 * G = dL/dS_t (starting at dS_T) and apply the chain rule to each line above,
 * last line first:
 *
 *     G   += q_t do_t^T                    (o_t = S_t^T q_t)
 *     dq_t = S_t do_t
 *     de   = G^T k_t                       (S_t = D + k e^T)
 *     dk_t = G e
 *     dv_t = beta_t de                     (e = beta (v - p))
 *     dbeta_t = de . (v_t - p)
 *     dp   = -beta_t de
 *     dD   = G + k_t dp^T                  (p = D^T k)
 *     dk_t += D dp
 *     dlog_alpha_t[i] = sum_j dD_ij D_ij   (D = Diag(exp(log_alpha)) S_{t-1})
 *     G    = Diag(alpha_t) dD              (dL/dS_{t-1})
 *
 * and dL/dS_0 = G after the first token.  Nothing is assumed about the
 * chunked form: this is the derivative of the token recurrence itself.
 *
 * The backward walk needs S_{t-1} for every token.  The forward pass keeps a
 * copy of S at the start of every SEG-token segment; the backward pass
 * re-runs one segment at a time from its copy (the same operations in the
 * same order, so the same bits) and walks it backwards.  Work is split over
 * (sequence, head) units, each of which produces its own tokens' gradients
 * completely, so the thread count changes no arithmetic.
 *
 * Storage: states as in kda_oracle.c, state[j][i] = S_ij (key index i
 * contiguous).  Inputs are cast exactly to fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { KDA_GRAD_F32 = 0, KDA_GRAD_BF16 = 1, KDA_GRAD_F64 = 2 };
enum { SEG = 64 };

static double elem(const void* base, int type, int64_t idx) {
  if (type == KDA_GRAD_F64) return ((const double*)base)[idx];
  if (type == KDA_GRAD_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;   /* bf16 */
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

typedef struct {
  const void *q, *k, *v, *log_alpha, *beta;
  int in_type, la_type;
  const int64_t* cu;
  const double *init_state, *d_o, *d_final;
  double *dq, *dk, *dv, *dla, *dbeta, *d_init;
  int H, K, V;          /* heads, key channels, value channels */
  int64_t n_units, next_unit;
} gjob_t;

/* Per-token inputs of (t, h) as fp64: a = exp(log_alpha), k, q, v, beta. */
static void token_inputs(const gjob_t* J, int64_t t, int h, double* a, double* kk, double* qq,
                         double* vv, double* beta) {
  const int64_t kb = (t * J->H + h) * J->K, vb = (t * J->H + h) * J->V;
  for (int i = 0; i < J->K; ++i) {
    a[i] = exp(elem(J->log_alpha, J->la_type, kb + i));
    kk[i] = elem(J->k, J->in_type, kb + i);
    qq[i] = elem(J->q, J->in_type, kb + i);
  }
  for (int j = 0; j < J->V; ++j) vv[j] = elem(J->v, J->in_type, vb + j);
  *beta = elem(J->beta, J->in_type, t * J->H + h);
}

/* One forward token on S (S[j*K + i] = S_ij): S <- D + k e^T.  Returns D in
 * Dout and p, e in pp, ee when they are non-NULL. */
static void forward_token(int K, int V, double* S, const double* a, const double* kk, const double* vv,
                          double beta, double* Dout, double* pp, double* ee) {
  for (int j = 0; j < V; ++j) {
    double* Sj = S + (int64_t)j * K;
    for (int i = 0; i < K; ++i) Sj[i] *= a[i];
    if (Dout) memcpy(Dout + (int64_t)j * K, Sj, sizeof(double) * (size_t)K);
    double p = 0.0;
    for (int i = 0; i < K; ++i) p += Sj[i] * kk[i];
    const double e = beta * (vv[j] - p);
    for (int i = 0; i < K; ++i) Sj[i] += kk[i] * e;
    if (pp) pp[j] = p;
    if (ee) ee[j] = e;
  }
}

typedef struct {
  double *S, *ckpt, *Dseg, *Sseg, *pseg, *eseg, *G, *a, *kk, *qq, *vv, *dD, *dp, *de;
} gbuf_t;

static void run_grad_unit(const gjob_t* J, int64_t u, gbuf_t* B) {
  const int H = J->H, K = J->K, V = J->V;
  const int h = (int)(u % H), n = (int)(u / H);
  const int64_t bos = J->cu[n], eos = J->cu[n + 1], L = eos - bos;
  const int64_t KV = (int64_t)K * V;
  const int64_t sbase = ((int64_t)n * H + h) * KV;
  const int64_t nseg = (L + SEG - 1) / SEG;

  /* forward: keep S at the start of every segment */
  for (int64_t x = 0; x < KV; ++x) B->S[x] = J->init_state ? J->init_state[sbase + x] : 0.0;
  double beta;
  for (int64_t s = 0; s < nseg; ++s) {
    memcpy(B->ckpt + s * KV, B->S, sizeof(double) * (size_t)KV);
    const int64_t t1 = bos + (s + 1) * SEG < eos ? bos + (s + 1) * SEG : eos;
    for (int64_t t = bos + s * SEG; t < t1; ++t) {
      token_inputs(J, t, h, B->a, B->kk, B->qq, B->vv, &beta);
      forward_token(K, V, B->S, B->a, B->kk, B->vv, beta, NULL, NULL, NULL);
    }
  }

  /* backward: G = dL/dS_t, from dL/dS_T */
  for (int64_t x = 0; x < KV; ++x) B->G[x] = J->d_final ? J->d_final[sbase + x] : 0.0;
  for (int64_t s = nseg - 1; s >= 0; --s) {
    const int64_t ta = bos + s * SEG;
    const int64_t tb = ta + SEG < eos ? ta + SEG : eos;
    /* re-run the segment, keeping D, S_t, p and e of every token */
    memcpy(B->S, B->ckpt + s * KV, sizeof(double) * (size_t)KV);
    for (int64_t t = ta; t < tb; ++t) {
      const int64_t r = t - ta;
      token_inputs(J, t, h, B->a, B->kk, B->qq, B->vv, &beta);
      forward_token(K, V, B->S, B->a, B->kk, B->vv, beta, B->Dseg + r * KV, B->pseg + r * V, B->eseg + r * V);
      memcpy(B->Sseg + r * KV, B->S, sizeof(double) * (size_t)KV);
    }
    for (int64_t t = tb - 1; t >= ta; --t) {
      const int64_t r = t - ta;
      const double* D = B->Dseg + r * KV;
      const double* St = B->Sseg + r * KV;
      const double* p = B->pseg + r * V;
      const double* e = B->eseg + r * V;
      token_inputs(J, t, h, B->a, B->kk, B->qq, B->vv, &beta);
      const double* dO = J->d_o + (t * H + h) * V;
      const int64_t kb = (t * H + h) * K;

      /* o_t = S_t^T q_t */
      for (int i = 0; i < K; ++i) {
        double acc = 0.0;
        for (int j = 0; j < V; ++j) acc += St[(int64_t)j * K + i] * dO[j];
        J->dq[kb + i] = acc;
      }
      for (int j = 0; j < V; ++j)
        for (int i = 0; i < K; ++i) B->G[(int64_t)j * K + i] += B->qq[i] * dO[j];
      /* S_t = D + k e^T */
      for (int j = 0; j < V; ++j) {
        double acc = 0.0;
        for (int i = 0; i < K; ++i) acc += B->G[(int64_t)j * K + i] * B->kk[i];
        B->de[j] = acc;
      }
      double db = 0.0;
      for (int j = 0; j < V; ++j) {
        J->dv[(t * H + h) * V + j] = beta * B->de[j];      /* e = beta (v - p) */
        db += B->de[j] * (B->vv[j] - p[j]);
        B->dp[j] = -beta * B->de[j];
      }
      J->dbeta[t * H + h] = db;
      for (int i = 0; i < K; ++i) {
        double acc1 = 0.0, acc2 = 0.0;
        for (int j = 0; j < V; ++j) {
          acc1 += B->G[(int64_t)j * K + i] * e[j];       /* from k e^T */
          acc2 += D[(int64_t)j * K + i] * B->dp[j];      /* from p = D^T k */
        }
        J->dk[kb + i] = acc1 + acc2;
      }
      /* dD = G + k dp^T, then D = Diag(alpha) S_{t-1} */
      for (int j = 0; j < V; ++j)
        for (int i = 0; i < K; ++i)
          B->dD[(int64_t)j * K + i] = B->G[(int64_t)j * K + i] + B->kk[i] * B->dp[j];
      for (int i = 0; i < K; ++i) {
        double acc = 0.0;
        for (int j = 0; j < V; ++j) acc += B->dD[(int64_t)j * K + i] * D[(int64_t)j * K + i];
        J->dla[kb + i] = acc;
      }
      for (int j = 0; j < V; ++j)
        for (int i = 0; i < K; ++i) B->G[(int64_t)j * K + i] = B->a[i] * B->dD[(int64_t)j * K + i];
    }
  }
  if (J->d_init) memcpy(J->d_init + sbase, B->G, sizeof(double) * (size_t)KV);
}

static void* grad_worker(void* arg) {
  gjob_t* J = (gjob_t*)arg;
  const int64_t KV = (int64_t)J->K * J->V;
  int64_t maxlen = 0;
  for (int64_t u = 0; u < J->n_units / J->H; ++u)
    if (J->cu[u + 1] - J->cu[u] > maxlen) maxlen = J->cu[u + 1] - J->cu[u];
  const int64_t nseg = (maxlen + SEG - 1) / SEG;
  gbuf_t B;
  memset(&B, 0, sizeof B);
  B.S = malloc(sizeof(double) * (size_t)KV);
  B.G = malloc(sizeof(double) * (size_t)KV);
  B.dD = malloc(sizeof(double) * (size_t)KV);
  B.ckpt = malloc(sizeof(double) * (size_t)(KV * (nseg > 0 ? nseg : 1)));
  B.Dseg = malloc(sizeof(double) * (size_t)(KV * SEG));
  B.Sseg = malloc(sizeof(double) * (size_t)(KV * SEG));
  B.pseg = malloc(sizeof(double) * (size_t)(J->V * SEG));
  B.eseg = malloc(sizeof(double) * (size_t)(J->V * SEG));
  B.a = malloc(sizeof(double) * (size_t)(3 * J->K + 3 * J->V));
  void* ret = NULL;
  if (!B.S || !B.G || !B.dD || !B.ckpt || !B.Dseg || !B.Sseg || !B.pseg || !B.eseg || !B.a) {
    ret = (void*)1;
  } else {
    B.kk = B.a + J->K;
    B.qq = B.kk + J->K;
    B.vv = B.qq + J->K;
    B.dp = B.vv + J->V;
    B.de = B.dp + J->V;
    for (;;) {
      int64_t u = __atomic_fetch_add(&J->next_unit, 1, __ATOMIC_RELAXED);
      if (u >= J->n_units) break;
      run_grad_unit(J, u, &B);
    }
  }
  free(B.S); free(B.G); free(B.dD); free(B.ckpt); free(B.Dseg); free(B.Sseg);
  free(B.pseg); free(B.eseg); free(B.a);
  return ret;
}

/*
 * Gradients of L = sum(d_o * o) + sum(d_final * final_state) for the varlen
 * prefill of kda_oracle_prefill (same inputs, same layouts):
 *   d_o        : fp64 [T, H, dv]
 *   d_final    : fp64 [num_seqs, H, dv, dk] or NULL (zero)
 *   dq, dk     : fp64 [T, H, dk];  dv : fp64 [T, H, dv]
 *   dla        : fp64 [T, H, dk]   (gradient w.r.t. log_alpha)
 *   dbeta      : fp64 [T, H]
 *   d_init     : fp64 [num_seqs, H, dv, dk] or NULL (not written)
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
int kda_oracle_prefill_grad(const void* q, const void* k, const void* v, const void* log_alpha,
                            const void* beta, int in_type, int la_type, const int64_t* cu_seqlens,
                            int num_seqs, const double* init_state, const double* d_o,
                            const double* d_final, double* dq, double* dk, double* dv, double* dla,
                            double* dbeta, double* d_init, int H, int K, int V, int nthreads) {
  if (!q || !k || !v || !log_alpha || !beta || !cu_seqlens || !d_o) return -1;
  if (!dq || !dk || !dv || !dla || !dbeta) return -1;
  if (num_seqs < 0 || H <= 0 || K <= 0 || V <= 0) return -1;
  if (in_type < 0 || in_type > 2 || (la_type != KDA_GRAD_F32 && la_type != KDA_GRAD_F64)) return -1;
  if (nthreads < 1) nthreads = 1;

  gjob_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta;
  J.in_type = in_type; J.la_type = la_type; J.cu = cu_seqlens;
  J.init_state = init_state; J.d_o = d_o; J.d_final = d_final;
  J.dq = dq; J.dk = dk; J.dv = dv; J.dla = dla; J.dbeta = dbeta; J.d_init = d_init;
  J.H = H; J.K = K; J.V = V;
  J.n_units = (int64_t)num_seqs * H;
  if (nthreads > J.n_units) nthreads = (int)(J.n_units > 0 ? J.n_units : 1);
  if (nthreads == 1) return grad_worker(&J) ? -2 : 0;

  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) return -2;
  int started = 0, rc = 0;
  for (; started < nthreads; ++started)
    if (pthread_create(&th[started], NULL, grad_worker, &J) != 0) break;
  if (started == 0) rc = grad_worker(&J) ? -2 : 0;
  for (int i = 0; i < started; ++i) {
    void* r = NULL;
    pthread_join(th[i], &r);
    if (r) rc = -2;
  }
  free(th);
  return rc;
}
