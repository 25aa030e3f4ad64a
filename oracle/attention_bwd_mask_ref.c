/*
 * oracle/attention_bwd_mask_ref.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * The gradients of exact attention under a general mask, in plain fp64, for the
 * test suite only.  It shares no code, header or constant with the GPU library
 * or with the other oracle files (each is complete on its own).
 *
 * The mask: for batch b, head h and query row r < N, key c is allowed when
 *   c < N,
 *   segment ids (if given, one array [B, N] shared by all heads) match:
 *     seg[b, c] == seg[b, r],
 *   and either c < prefix, or
 *     (window_left  < 0 or c >= r - window_left) and
 *     (window_right < 0 or c <= r + window_right).
 * A causal mask is window_right = 0.  The forward over the allowed keys A_r is
 *   s_rc = scale * q_r . k_c,   p_r = softmax_c(s_rc),   o_r = sum_c p_rc v_c,
 * and masked pairs have p = 0 (a 0 / -inf term added to the scores before the
 * softmax).  Given dO, the chain rule through the three stages gives
 *   dV   = P^T dO,   dP = dO V^T,   D_r = sum_c P_rc dP_rc,
 *   dS   = P o (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q,
 * where masked pairs contribute nothing (P = 0, so dS = 0).  A row with no
 * allowed key (none occurs for these masks: c = r is always allowed) gets zero
 * gradients and D = 0.
 *
 * Sources:
 *  - The mask as a 0 / -inf score term, covering sliding windows, document
 *    boundaries and prefix language models: "Flash Attention 2", section
 *    "Causal masking".  The exact shape of each mask is not spelled out there;
 *    the reading above is the plain one.
 *  - The softmax gradient dS = P o (dP - D): "6.2 FlashAttention V2 in depth",
 *    section 7.3; recomputing P instead of storing it: same page, section 7.1,
 *    and "Flash Attention: Memory-Efficient Attention at Scale", section
 *    "Recomputation in the backward pass".  Here P is computed from its
 *    definition.
 *
 * Each worker owns whole (b, h) slices and walks their rows one at a time;
 * there is no tiling along keys and no online softmax.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

typedef struct {
  const double *q, *k, *v, *dout; /* [N, d] of this head */
  const int32_t* seg;             /* [N] of this batch, or NULL */
  double *dq, *dk, *dv;           /* [N, d] of this head */
  double* delta;                  /* [N] of this head, or NULL */
  int64_t N, d, wl, wr, prefix;
  double scale;
} bwdm_task;

static int bwdm_allowed(const bwdm_task* t, int64_t r, int64_t c) {
  if (c >= t->N) return 0;
  if (t->seg && t->seg[c] != t->seg[r]) return 0;
  if (c < t->prefix) return 1;
  if (t->wl >= 0 && c < r - t->wl) return 0;
  if (t->wr >= 0 && c > r + t->wr) return 0;
  return 1;
}

/* One (b, h) slice; p and dp hold one row of N doubles each. */
static void bwdm_head(const bwdm_task* t, double* p, double* dp) {
  const int64_t N = t->N, d = t->d;
  for (int64_t u = 0; u < N * d; ++u) {
    t->dk[u] = 0.0;
    t->dv[u] = 0.0;
  }
  for (int64_t r = 0; r < N; ++r) {
    const double* qr = t->q + r * d;
    const double* gr = t->dout + r * d;
    double* dqr = t->dq + r * d;
    for (int64_t u = 0; u < d; ++u) dqr[u] = 0.0;
    /* scores of the allowed keys and their maximum */
    double m = -INFINITY;
    for (int64_t c = 0; c < N; ++c) {
      if (!bwdm_allowed(t, r, c)) continue;
      double acc = 0.0;
      for (int64_t u = 0; u < d; ++u) acc += qr[u] * t->k[c * d + u];
      p[c] = t->scale * acc;
      if (p[c] > m) m = p[c];
    }
    if (m == -INFINITY) { /* no allowed key */
      if (t->delta) t->delta[r] = 0.0;
      continue;
    }
    double l = 0.0;
    for (int64_t c = 0; c < N; ++c)
      if (bwdm_allowed(t, r, c)) l += exp(p[c] - m);
    /* P, dP = dO V^T and D = rowsum(P o dP) over the allowed keys */
    double D = 0.0;
    for (int64_t c = 0; c < N; ++c) {
      if (!bwdm_allowed(t, r, c)) continue;
      p[c] = exp(p[c] - m) / l;
      double acc = 0.0;
      for (int64_t u = 0; u < d; ++u) acc += gr[u] * t->v[c * d + u];
      dp[c] = acc;
      D += p[c] * acc;
    }
    if (t->delta) t->delta[r] = D;
    /* dS = P o (dP - D); the row's dQ and its share of dK and dV */
    for (int64_t c = 0; c < N; ++c) {
      if (!bwdm_allowed(t, r, c)) continue;
      const double ds = p[c] * (dp[c] - D);
      const double* kc = t->k + c * d;
      double* dkc = t->dk + c * d;
      double* dvc = t->dv + c * d;
      for (int64_t u = 0; u < d; ++u) {
        dqr[u] += t->scale * ds * kc[u];
        dkc[u] += t->scale * ds * qr[u];
        dvc[u] += p[c] * gr[u];
      }
    }
  }
}

typedef struct {
  bwdm_task* tasks;
  int64_t ntasks, next, N;
  pthread_mutex_t lock;
  int failed;
} bwdm_pool;

static void* bwdm_worker(void* arg) {
  bwdm_pool* pool = (bwdm_pool*)arg;
  double* p = (double*)malloc(sizeof(double) * (size_t)pool->N);
  double* dp = (double*)malloc(sizeof(double) * (size_t)pool->N);
  if (!p || !dp) {
    free(p);
    free(dp);
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
    bwdm_head(&pool->tasks[my], p, dp);
  }
  free(p);
  free(dp);
  return NULL;
}

/*
 * Gradients over [B, H, N, d] row-major fp64 arrays under the mask above: dout
 * is dO; dq, dk, dv are written in full; delta ([B, H, N], may be NULL) receives
 * D; seg is NULL or [B, N].  Returns 0 on success, -1 on bad sizes, -2 when
 * memory runs out.
 */
int oracle_attention_bwd_masked_f64(const double* q, const double* k, const double* v, const double* dout,
                                    double* dq, double* dk, double* dv, double* delta, int64_t B, int64_t H,
                                    int64_t N, int64_t d, int64_t window_left, int64_t window_right,
                                    int64_t prefix, const int32_t* seg, double scale, int nthreads) {
  if (B < 0 || H < 0 || N < 0 || d < 1 || prefix < 0) return -1;
  if (B == 0 || H == 0 || N == 0) return 0;
  const int64_t ntasks = B * H;
  bwdm_task* tasks = (bwdm_task*)malloc(sizeof(bwdm_task) * (size_t)ntasks);
  if (!tasks) return -2;
  for (int64_t bh = 0; bh < ntasks; ++bh) {
    bwdm_task* t = &tasks[bh];
    const int64_t off = bh * N * d;
    t->q = q + off;
    t->k = k + off;
    t->v = v + off;
    t->dout = dout + off;
    t->seg = seg ? seg + (bh / H) * N : NULL;
    t->dq = dq + off;
    t->dk = dk + off;
    t->dv = dv + off;
    t->delta = delta ? delta + bh * N : NULL;
    t->N = N;
    t->d = d;
    t->wl = window_left;
    t->wr = window_right;
    t->prefix = prefix;
    t->scale = scale;
  }
  bwdm_pool pool;
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
    if (pthread_create(&th[i], NULL, bwdm_worker, &pool) == 0) ++started;
  if (started == 0) bwdm_worker(&pool);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&pool.lock);
  free(tasks);
  return pool.failed ? -2 : 0;
}
