/*
 * oracle/attention_decode_ref.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * Exact attention of a few new query rows against a key/value cache, in plain
 * fp64, for the test suite only.  It shares no code with the GPU library or with
 * the other oracle files.
 *
 * For batch b, head h and new query i < Mq, with the cache holding len_b valid
 * rows (len_b = seqlens[b], or Nk when no lengths are given), key c is allowed
 * when c < len_b and, under the causal flag, c <= len_b - Mq + i: the Mq new
 * rows are the last Mq positions of a sequence of len_b tokens, so query i sits
 * at position len_b - Mq + i and sees the keys up to its own position.  Over the
 * allowed keys A_i:
 *   s_ic = scale * q_i . k_c,   o_i = sum_c softmax_c(s_ic) v_c,
 *   lse_i = log sum_c exp(s_ic)  (natural log).
 * A query with no allowed key (len_b = 0, or len_b < Mq under the causal flag)
 * gets o_i = 0 and lse_i = -inf.
 *
 * Sources: the definition of attention (scores, row softmax, P.V) is that of
 * "Flash Attention: Memory-Efficient Attention at Scale", section "A quick
 * recap of standard attention"; the same page, section "Common misconceptions",
 * names single-token decoding (one query row against the cached keys and
 * values) as the regime that needs its own kernels; the causal mask as "each
 * position sees itself and earlier positions" is that of "Flash Attention 2",
 * section "Causal masking".  Where the new rows sit in the sequence (the last
 * Mq positions) is not spelled out there; the reading above is the plain one
 * for generation, where the new tokens follow the cached ones.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

typedef struct {
  const double *q, *k, *v; /* q: [Mq, d] of this head; k, v: [Nk, d] */
  double *o, *lse;         /* [Mq, d], [Mq] */
  int64_t Mq, len, d;
  int causal;
  double scale;
} decode_task;

static void decode_head(const decode_task* t, double* s) {
  const int64_t d = t->d;
  for (int64_t i = 0; i < t->Mq; ++i) {
    int64_t last = t->len - 1; /* last allowed key */
    if (t->causal) last = t->len - t->Mq + i;
    const double* qi = t->q + i * d;
    double* oi = t->o + i * d;
    for (int64_t u = 0; u < d; ++u) oi[u] = 0.0;
    if (last < 0) {
      t->lse[i] = -INFINITY;
      continue;
    }
    double m = -INFINITY;
    for (int64_t c = 0; c <= last; ++c) {
      double acc = 0.0;
      for (int64_t u = 0; u < d; ++u) acc += qi[u] * t->k[c * d + u];
      s[c] = t->scale * acc;
      if (s[c] > m) m = s[c];
    }
    double l = 0.0;
    for (int64_t c = 0; c <= last; ++c) l += exp(s[c] - m);
    for (int64_t c = 0; c <= last; ++c) {
      const double p = exp(s[c] - m) / l;
      for (int64_t u = 0; u < d; ++u) oi[u] += p * t->v[c * d + u];
    }
    t->lse[i] = m + log(l);
  }
}

typedef struct {
  decode_task* tasks;
  int64_t ntasks, next, Nk;
  pthread_mutex_t lock;
  int failed;
} decode_pool;

static void* decode_worker(void* arg) {
  decode_pool* pool = (decode_pool*)arg;
  double* s = (double*)malloc(sizeof(double) * (size_t)(pool->Nk > 0 ? pool->Nk : 1));
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
    decode_head(&pool->tasks[my], s);
  }
  free(s);
  return NULL;
}

/*
 * q: [B, H, Mq, d]; k, v: [B, H, Nk, d]; seqlens: [B] (each in [0, Nk]) or NULL
 * for Nk; o: [B, H, Mq, d]; lse: [B, H, Mq].  Returns 0, -1 on bad sizes or a
 * length outside [0, Nk], -2 when memory runs out.
 */
int oracle_attention_decode_f64(const double* q, const double* k, const double* v, const int32_t* seqlens,
                                double* o, double* lse, int64_t B, int64_t H, int64_t Mq, int64_t Nk, int64_t d,
                                int causal, double scale, int nthreads) {
  if (B < 0 || H < 0 || Mq < 0 || Nk < 0 || d < 1) return -1;
  if (seqlens)
    for (int64_t b = 0; b < B; ++b)
      if (seqlens[b] < 0 || seqlens[b] > Nk) return -1;
  if (B == 0 || H == 0 || Mq == 0) return 0;
  const int64_t ntasks = B * H;
  decode_task* tasks = (decode_task*)malloc(sizeof(decode_task) * (size_t)ntasks);
  if (!tasks) return -2;
  for (int64_t bh = 0; bh < ntasks; ++bh) {
    decode_task* t = &tasks[bh];
    t->q = q + bh * Mq * d;
    t->k = k + bh * Nk * d;
    t->v = v + bh * Nk * d;
    t->o = o + bh * Mq * d;
    t->lse = lse + bh * Mq;
    t->Mq = Mq;
    t->len = seqlens ? seqlens[bh / H] : Nk;
    t->d = d;
    t->causal = causal;
    t->scale = scale;
  }
  decode_pool pool;
  pool.tasks = tasks;
  pool.ntasks = ntasks;
  pool.next = 0;
  pool.Nk = Nk;
  pool.failed = 0;
  pthread_mutex_init(&pool.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > ntasks) nthreads = (int)ntasks;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  for (int i = 0; th && i < nthreads; ++i)
    if (pthread_create(&th[i], NULL, decode_worker, &pool) == 0) ++started;
  if (started == 0) decode_worker(&pool);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&pool.lock);
  free(tasks);
  return pool.failed ? -2 : 0;
}
