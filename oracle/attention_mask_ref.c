/*
 * oracle/attention_mask_ref.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * Exact attention under a general mask, in plain fp64, for the test suite only.
 * It shares no code with the GPU library or with the other oracle files.
 *
 * For batch b, head h and query row r < N, key c is allowed when
 *   c < N,
 *   segment ids (if given, one array [B, N] shared by all heads) match:
 *     seg[b, c] == seg[b, r],
 *   and either c < prefix (a prefix visible to every query), or c lies in the
 *   window around r:
 *     (window_left  < 0 or c >= r - window_left) and
 *     (window_right < 0 or c <= r + window_right).
 * A causal mask is window_right = 0.  Over the allowed keys A_r:
 *   s_rc = scale * q_r . k_c,   o_r = sum_c softmax_c(s_rc) v_c,
 *   lse_r = log sum_c exp(s_rc)  (natural log).
 * A row with no allowed key gets o_r = 0 and lse_r = -inf (none occurs for the
 * masks above, which always allow c = r).
 *
 * Sources: "Flash Attention 2", section "Causal masking": a mask is a 0 / -inf
 * term added to the scores before the softmax, so masked keys carry zero
 * weight, and the same scheme covers sliding windows, document boundaries and
 * prefix language models; the definition of attention itself follows
 * "Flash Attention: Memory-Efficient Attention at Scale", section "A quick
 * recap of standard attention".  The exact shape of each mask (which keys a
 * window, a prefix or a document boundary admits) is not spelled out there;
 * the reading above is the plain one.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

typedef struct {
  const double *q, *k, *v;
  const int32_t* seg; /* [N] of this batch, or NULL */
  double *o, *lse;    /* [N, d], [N] of this head */
  int64_t N, d, wl, wr, prefix;
  double scale;
} mask_task;

static int allowed(const mask_task* t, int64_t r, int64_t c) {
  if (c >= t->N) return 0;
  if (t->seg && t->seg[c] != t->seg[r]) return 0;
  if (c < t->prefix) return 1;
  if (t->wl >= 0 && c < r - t->wl) return 0;
  if (t->wr >= 0 && c > r + t->wr) return 0;
  return 1;
}

static void mask_head(const mask_task* t, double* s) {
  const int64_t N = t->N, d = t->d;
  for (int64_t r = 0; r < N; ++r) {
    const double* qr = t->q + r * d;
    double m = -INFINITY;
    for (int64_t c = 0; c < N; ++c) {
      if (!allowed(t, r, c)) continue;
      double acc = 0.0;
      for (int64_t u = 0; u < d; ++u) acc += qr[u] * t->k[c * d + u];
      s[c] = t->scale * acc;
      m = s[c] > m ? s[c] : m;
    }
    double* orow = t->o + r * d;
    for (int64_t u = 0; u < d; ++u) orow[u] = 0.0;
    if (m == -INFINITY) {
      t->lse[r] = -INFINITY;
      continue;
    }
    double l = 0.0;
    for (int64_t c = 0; c < N; ++c)
      if (allowed(t, r, c)) l += exp(s[c] - m);
    for (int64_t c = 0; c < N; ++c) {
      if (!allowed(t, r, c)) continue;
      const double p = exp(s[c] - m) / l;
      for (int64_t u = 0; u < d; ++u) orow[u] += p * t->v[c * d + u];
    }
    t->lse[r] = m + log(l);
  }
}

typedef struct {
  mask_task* tasks;
  int64_t ntasks, next, N;
  pthread_mutex_t lock;
  int failed;
} mask_pool;

static void* mask_worker(void* arg) {
  mask_pool* pool = (mask_pool*)arg;
  double* s = (double*)malloc(sizeof(double) * (size_t)(pool->N > 0 ? pool->N : 1));
  if (!s) {
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
    mask_head(&pool->tasks[my], s);
  }
  free(s);
  return NULL;
}

/*
 * q, k, v, o: [B, H, N, d]; lse: [B, H, N]; seg: [B, N] or NULL.  Returns 0,
 * -1 on bad sizes, -2 when memory runs out.
 */
int oracle_attention_masked_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                                int64_t B, int64_t H, int64_t N, int64_t d, int64_t window_left,
                                int64_t window_right, int64_t prefix, const int32_t* seg, double scale,
                                int nthreads) {
  if (B < 0 || H < 0 || N < 0 || d < 1) return -1;
  if (B == 0 || H == 0 || N == 0) return 0;
  const int64_t ntasks = B * H;
  mask_task* tasks = (mask_task*)malloc(sizeof(mask_task) * (size_t)ntasks);
  if (!tasks) return -2;
  for (int64_t bh = 0; bh < ntasks; ++bh) {
    mask_task* t = &tasks[bh];
    const int64_t b = bh / H;
    t->q = q + bh * N * d;
    t->k = k + bh * N * d;
    t->v = v + bh * N * d;
    t->seg = seg ? seg + b * N : NULL;
    t->o = o + bh * N * d;
    t->lse = lse + bh * N;
    t->N = N;
    t->d = d;
    t->wl = window_left;
    t->wr = window_right;
    t->prefix = prefix;
    t->scale = scale;
  }
  mask_pool pool;
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
    if (pthread_create(&th[i], NULL, mask_worker, &pool) == 0) ++started;
  if (started == 0) mask_worker(&pool);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&pool.lock);
  free(tasks);
  return pool.failed ? -2 : 0;
}
