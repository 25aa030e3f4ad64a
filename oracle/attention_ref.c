/*
 * oracle/attention_ref.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * A plain, slow fp64 CPU implementation of exact (standard) attention.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header or constant with the GPU library.
 *
 * What it computes, for every batch b, head h and query row r < N, over the set
 * A_r of allowed keys (all c < N; with a causal mask only c <= r):
 *
 *   s_rc = scale * sum_t q[r,t] k[c,t]                 (scores)
 *   p_rc = exp(s_rc - m_r) / sum_{c' in A_r} exp(s_rc' - m_r),   m_r = max_c s_rc
 *   o[r,:] = sum_{c in A_r} p_rc v[c,:]                (output)
 *   lse_r = m_r + log(sum_{c in A_r} exp(s_rc - m_r))  (natural-log logsumexp)
 *
 * Sources:
 *  - "Flash Attention: Memory-Efficient Attention at Scale" (Lesson 6.6), section
 *    "A quick recap of standard attention": the three stages scores -> row softmax
 *    -> P.V, with scores divided by sqrt(d).  Here the multiplier is the explicit
 *    `scale` argument.
 *  - "Flash Attention 2", section "Standard Attention" (S = QK^T, row softmax,
 *    O = PV; each softmax row sums to one) and section "Causal masking" (mask
 *    M_ij = 0 for j <= i and -inf for j > i, so masked keys carry zero weight).
 *    Masked keys are left out of A_r, which is the same thing as adding -inf.
 *  - "6.2 FlashAttention V2 in depth", section 6.1 (the pseudocode returns the
 *    per-row statistic L = m + log l) and section 7.1 (L is the row-wise
 *    logsumexp of the scaled, masked scores).
 *
 * The three stages run one after another on a block of rows; rows are
 * independent in standard attention, so splitting the rows into blocks only
 * bounds memory (a causal 16k x 16k score block per head would be 2 GiB).
 * There is no online softmax, no running rescale and no tiling along keys.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ROW_BLOCK 64

/* One unit of work: a block of query rows of one (b, h) slice. */
typedef struct {
  const double* q; /* [N, d] of this head */
  const double* k; /* [N, d] */
  const double* v; /* [N, d] */
  double* o;       /* output rows, row-major, d per row */
  double* lse;     /* output statistic, one per row */
  const int64_t* rows; /* query row indices (length nrows) */
  int64_t nrows;
  int64_t N, d;
  int causal;
  double scale;
} oracle_task;

/* Stage 1..3 for one block of rows; `S` has room for nrows * N doubles. */
static void oracle_rows(const oracle_task* t, double* S) {
  const int64_t N = t->N, d = t->d;
  /* Stage 1: scores for the allowed keys of every row in the block. */
  for (int64_t i = 0; i < t->nrows; ++i) {
    const int64_t r = t->rows[i];
    const int64_t ncols = t->causal ? r + 1 : N; /* allowed keys are 0..ncols-1 */
    const double* qr = t->q + r * d;
    double* Sr = S + i * N;
    for (int64_t c = 0; c < ncols; ++c) {
      const double* kc = t->k + c * d;
      double acc = 0.0;
      for (int64_t u = 0; u < d; ++u) acc += qr[u] * kc[u];
      Sr[c] = t->scale * acc;
    }
  }
  /* Stage 2: row softmax (max, sum of exponentials, normalised weights). */
  double* stat_m = (double*)malloc(sizeof(double) * (size_t)t->nrows);
  double* stat_l = (double*)malloc(sizeof(double) * (size_t)t->nrows);
  for (int64_t i = 0; i < t->nrows; ++i) {
    const int64_t r = t->rows[i];
    const int64_t ncols = t->causal ? r + 1 : N;
    double* Sr = S + i * N;
    double m = -INFINITY;
    for (int64_t c = 0; c < ncols; ++c) m = Sr[c] > m ? Sr[c] : m;
    double l = 0.0;
    for (int64_t c = 0; c < ncols; ++c) l += exp(Sr[c] - m);
    for (int64_t c = 0; c < ncols; ++c) Sr[c] = exp(Sr[c] - m) / l; /* now P */
    stat_m[i] = m;
    stat_l[i] = l;
  }
  /* Stage 3: O = P V, and the logsumexp statistic. */
  for (int64_t i = 0; i < t->nrows; ++i) {
    const int64_t r = t->rows[i];
    const int64_t ncols = t->causal ? r + 1 : N;
    const double* Pr = S + i * N;
    double* orow = t->o + i * d;
    for (int64_t u = 0; u < d; ++u) orow[u] = 0.0;
    for (int64_t c = 0; c < ncols; ++c) {
      const double p = Pr[c];
      const double* vc = t->v + c * d;
      for (int64_t u = 0; u < d; ++u) orow[u] += p * vc[u];
    }
    t->lse[i] = stat_m[i] + log(stat_l[i]);
  }
  free(stat_m);
  free(stat_l);
}

typedef struct {
  oracle_task* tasks;
  int64_t ntasks;
  int64_t next;
  int64_t N;
  pthread_mutex_t lock;
  int failed;
} oracle_pool;

static void* oracle_worker(void* arg) {
  oracle_pool* pool = (oracle_pool*)arg;
  double* S = (double*)malloc(sizeof(double) * (size_t)ORACLE_ROW_BLOCK * (size_t)pool->N);
  if (!S) {
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
    oracle_rows(&pool->tasks[my], S);
  }
  free(S);
  return NULL;
}

static int oracle_run(oracle_task* tasks, int64_t ntasks, int64_t N, int nthreads) {
  oracle_pool pool;
  pool.tasks = tasks;
  pool.ntasks = ntasks;
  pool.next = 0;
  pool.N = N;
  pool.failed = 0;
  pthread_mutex_init(&pool.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > ntasks) nthreads = (int)(ntasks > 0 ? ntasks : 1);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, oracle_worker, &pool) == 0) ++started;
  }
  if (started == 0) oracle_worker(&pool);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&pool.lock);
  return pool.failed ? -2 : 0;
}

/*
 * Full attention over [B, H, N, d] row-major fp64 arrays.
 * o: [B, H, N, d], lse: [B, H, N].  Returns 0 on success, -1 on bad sizes,
 * -2 when memory runs out.
 */
int oracle_attention_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                         int64_t B, int64_t H, int64_t N, int64_t d, int causal, double scale,
                         int nthreads) {
  if (B < 0 || H < 0 || N < 0 || d < 1) return -1;
  if (B == 0 || H == 0 || N == 0) return 0;
  const int64_t nblk = (N + ORACLE_ROW_BLOCK - 1) / ORACLE_ROW_BLOCK;
  const int64_t ntasks = B * H * nblk;
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  oracle_task* tasks = (oracle_task*)malloc(sizeof(oracle_task) * (size_t)ntasks);
  if (!rows || !tasks) {
    free(rows);
    free(tasks);
    return -2;
  }
  for (int64_t r = 0; r < N; ++r) rows[r] = r;
  int64_t n = 0;
  for (int64_t bh = 0; bh < B * H; ++bh) {
    for (int64_t blk = 0; blk < nblk; ++blk) {
      const int64_t r0 = blk * ORACLE_ROW_BLOCK;
      const int64_t r1 = r0 + ORACLE_ROW_BLOCK < N ? r0 + ORACLE_ROW_BLOCK : N;
      oracle_task* t = &tasks[n++];
      t->q = q + bh * N * d;
      t->k = k + bh * N * d;
      t->v = v + bh * N * d;
      t->o = o + (bh * N + r0) * d;
      t->lse = lse + bh * N + r0;
      t->rows = rows + r0;
      t->nrows = r1 - r0;
      t->N = N;
      t->d = d;
      t->causal = causal;
      t->scale = scale;
    }
  }
  const int rc = oracle_run(tasks, ntasks, N, nthreads);
  free(tasks);
  free(rows);
  return rc;
}

/*
 * Selected query rows of one head: q, k, v are [N, d]; rows holds R row indices
 * in [0, N).  o: [R, d], lse: [R].  Used to check sampled outputs of large
 * problems one row at a time.  Returns 0, -1 on bad arguments, -2 on no memory.
 */
int oracle_attention_rows_f64(const double* q, const double* k, const double* v,
                              const int64_t* rows, int64_t R, double* o, double* lse,
                              int64_t N, int64_t d, int causal, double scale, int nthreads) {
  if (R < 0 || N < 1 || d < 1) return -1;
  for (int64_t i = 0; i < R; ++i)
    if (rows[i] < 0 || rows[i] >= N) return -1;
  if (R == 0) return 0;
  const int64_t ntasks = (R + ORACLE_ROW_BLOCK - 1) / ORACLE_ROW_BLOCK;
  oracle_task* tasks = (oracle_task*)malloc(sizeof(oracle_task) * (size_t)ntasks);
  if (!tasks) return -2;
  for (int64_t n = 0; n < ntasks; ++n) {
    const int64_t i0 = n * ORACLE_ROW_BLOCK;
    const int64_t i1 = i0 + ORACLE_ROW_BLOCK < R ? i0 + ORACLE_ROW_BLOCK : R;
    oracle_task* t = &tasks[n];
    t->q = q;
    t->k = k;
    t->v = v;
    t->o = o + i0 * d;
    t->lse = lse + i0;
    t->rows = rows + i0;
    t->nrows = i1 - i0;
    t->N = N;
    t->d = d;
    t->causal = causal;
    t->scale = scale;
  }
  const int rc = oracle_run(tasks, ntasks, N, nthreads);
  free(tasks);
  return rc;
}
