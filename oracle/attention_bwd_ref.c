/*
 * oracle/attention_bwd_ref.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * The gradients of exact (standard) attention in plain fp64, for the test suite
 * only.  It shares no code, header or constant with the GPU library (nor with
 * the forward oracle beside it: each file is complete on its own).
 *
 * Forward (as defined in attention_ref.c): for each (b, h) and query row r, over
 * the allowed keys A_r (all c < N; with a causal mask only c <= r),
 *   s_rc = scale * q_r . k_c,   p_r = softmax_c(s_rc),   o_r = sum_c p_rc v_c.
 * Given the gradient dO of a scalar loss with respect to O, the gradients are
 * the chain rule through those three stages:
 *   dV   = P^T dO                                  (o_r is linear in v_c)
 *   dP   = dO V^T                                  (dP_rc = dO_r . v_c)
 *   D_r  = sum_c P_rc dP_rc                        (row-wise)
 *   dS   = P o (dP - D)                            (softmax Jacobian, row by row)
 *   dQ   = scale * dS K,   dK = scale * dS^T Q     (s_rc = scale * q_r . k_c)
 * Masked pairs have P = 0, hence dS = 0: they contribute to nothing.
 *
 * Sources:
 *  - "6.2 FlashAttention V2 in depth", section 7.3: the softmax gradient
 *    dS = P o (dP - D) with D the row sum of dP o P (which equals the row sum
 *    of dO o O; the GPU path uses that second form, this oracle the first).
 *  - Same page, section 7.1: the backward pass recovers P from the saved
 *    logsumexp as exp(S - L).  Here P is recomputed from its definition.
 *  - "Flash Attention: Memory-Efficient Attention at Scale", section
 *    "Recomputation in the backward pass": the score tiles are recomputed from
 *    Q and K rather than stored.
 *  - The forward stages themselves: "Flash Attention: Memory-Efficient
 *    Attention at Scale", section "A quick recap of standard attention", and
 *    "Flash Attention 2", sections "Standard Attention" and "Causal masking".
 *
 * Each worker owns whole (b, h) slices and walks their query rows in blocks:
 * the rows of a block give their dQ rows directly and add their share to the
 * slice's dK and dV.  Blocking bounds memory only; there is no tiling along
 * keys and no online softmax.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define BWD_ROW_BLOCK 64

typedef struct {
  const double *q, *k, *v, *dout; /* [N, d] of this head */
  double *dq, *dk, *dv;           /* [N, d] of this head */
  double* delta;                  /* [N] of this head, or NULL */
  int64_t N, d;
  int causal;
  double scale;
} bwd_task;

/* One (b, h) slice.  P and dP are blocks of nrows x N doubles. */
static void bwd_head(const bwd_task* t, double* P, double* dP) {
  const int64_t N = t->N, d = t->d;
  for (int64_t u = 0; u < N * d; ++u) {
    t->dk[u] = 0.0;
    t->dv[u] = 0.0;
  }
  for (int64_t r0 = 0; r0 < N; r0 += BWD_ROW_BLOCK) {
    const int64_t r1 = r0 + BWD_ROW_BLOCK < N ? r0 + BWD_ROW_BLOCK : N;
    for (int64_t r = r0; r < r1; ++r) {
      const int64_t ncols = t->causal ? r + 1 : N; /* allowed keys 0..ncols-1 */
      const double* qr = t->q + r * d;
      const double* gr = t->dout + r * d;
      double* Pr = P + (r - r0) * N;
      double* dPr = dP + (r - r0) * N;
      /* Scores, then the row softmax. */
      double m = -INFINITY;
      for (int64_t c = 0; c < ncols; ++c) {
        const double* kc = t->k + c * d;
        double acc = 0.0;
        for (int64_t u = 0; u < d; ++u) acc += qr[u] * kc[u];
        Pr[c] = t->scale * acc;
        m = Pr[c] > m ? Pr[c] : m;
      }
      double l = 0.0;
      for (int64_t c = 0; c < ncols; ++c) l += exp(Pr[c] - m);
      for (int64_t c = 0; c < ncols; ++c) Pr[c] = exp(Pr[c] - m) / l;
      /* dP = dO V^T on the allowed keys; D = rowsum(P o dP). */
      double D = 0.0;
      for (int64_t c = 0; c < ncols; ++c) {
        const double* vc = t->v + c * d;
        double acc = 0.0;
        for (int64_t u = 0; u < d; ++u) acc += gr[u] * vc[u];
        dPr[c] = acc;
        D += Pr[c] * acc;
      }
      if (t->delta) t->delta[r] = D;
      /* dS = P o (dP - D), kept in place of dP. */
      for (int64_t c = 0; c < ncols; ++c) dPr[c] = Pr[c] * (dPr[c] - D);
      /* dQ row, and this row's share of dK and dV. */
      double* dqr = t->dq + r * d;
      for (int64_t u = 0; u < d; ++u) dqr[u] = 0.0;
      for (int64_t c = 0; c < ncols; ++c) {
        const double* kc = t->k + c * d;
        const double ds = dPr[c];
        const double p = Pr[c];
        double* dkc = t->dk + c * d;
        double* dvc = t->dv + c * d;
        for (int64_t u = 0; u < d; ++u) {
          dqr[u] += t->scale * ds * kc[u];
          dkc[u] += t->scale * ds * qr[u];
          dvc[u] += p * gr[u];
        }
      }
    }
  }
}

typedef struct {
  bwd_task* tasks;
  int64_t ntasks, next, N;
  pthread_mutex_t lock;
  int failed;
} bwd_pool;

static void* bwd_worker(void* arg) {
  bwd_pool* pool = (bwd_pool*)arg;
  const size_t blk = sizeof(double) * (size_t)BWD_ROW_BLOCK * (size_t)pool->N;
  double* P = (double*)malloc(blk);
  double* dP = (double*)malloc(blk);
  if (!P || !dP) {
    free(P);
    free(dP);
    pthread_mutex_lock(&pool->lock);
    pool->failed = 1;
    pthread_mutex_unlock(&pool->lock);
    return NULL;
  }
  for (;;) {
    pthread_mutex_lock(&pool->lock);
    const int64_t my = pool->next++;
    pthread_mutex_unlock(&pool->lock);
    if (my >= pool->ntasks) break;
    bwd_head(&pool->tasks[my], P, dP);
  }
  free(P);
  free(dP);
  return NULL;
}

/*
 * Gradients over [B, H, N, d] row-major fp64 arrays: dout is dO; dq, dk, dv are
 * written in full; delta ([B, H, N], may be NULL) receives D.  Returns 0 on
 * success, -1 on bad sizes, -2 when memory runs out.
 */
int oracle_attention_bwd_f64(const double* q, const double* k, const double* v, const double* dout,
                             double* dq, double* dk, double* dv, double* delta, int64_t B, int64_t H,
                             int64_t N, int64_t d, int causal, double scale, int nthreads) {
  if (B < 0 || H < 0 || N < 0 || d < 1) return -1;
  if (B == 0 || H == 0 || N == 0) return 0;
  const int64_t ntasks = B * H;
  bwd_task* tasks = (bwd_task*)malloc(sizeof(bwd_task) * (size_t)ntasks);
  if (!tasks) return -2;
  for (int64_t bh = 0; bh < ntasks; ++bh) {
    bwd_task* t = &tasks[bh];
    const int64_t off = bh * N * d;
    t->q = q + off;
    t->k = k + off;
    t->v = v + off;
    t->dout = dout + off;
    t->dq = dq + off;
    t->dk = dk + off;
    t->dv = dv + off;
    t->delta = delta ? delta + bh * N : NULL;
    t->N = N;
    t->d = d;
    t->causal = causal;
    t->scale = scale;
  }
  bwd_pool pool;
  pool.tasks = tasks;
  pool.ntasks = ntasks;
  pool.next = 0;
  pool.N = N;
  pool.failed = 0;
  pthread_mutex_init(&pool.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > ntasks) nthreads = (int)ntasks;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  for (int i = 0; th && i < nthreads; ++i)
    if (pthread_create(&th[i], NULL, bwd_worker, &pool) == 0) ++started;
  if (started == 0) bwd_worker(&pool);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&pool.lock);
  free(tasks);
  return pool.failed ? -2 : 0;
}
