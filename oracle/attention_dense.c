/*
 * Dense fp64 attention oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code
 * with the GPU library and must never be called from the product path.
 *
 * What it computes is the plain definition of attention that the dense
 * reference of the aiml.sh page "Speed up long contexts with FlashAttention"
 * (lab.py, function standard_attention) writes out: for each head and each
 * query row i,
 *
 *   allowed keys A(i) = {0..i} when causal, {0..S-1} otherwise
 *   s_ij  = (q_i . k_j) * scale                       for j in A(i)
 *   m_i   = max_j s_ij
 *   p_ij  = exp(s_ij - m_i) / sum_j exp(s_ij - m_i)
 *   o_i   = sum_j p_ij v_j
 *   lse_i = m_i + log(sum_j exp(s_ij - m_i))
 *
 * The score row and the probability row of each query are materialised in
 * full before the product with V, as that reference does; there is no tiling
 * and no online rescaling.  The log-sum-exp is not on the pages; it is the
 * natural log of the softmax denominator including the scale (this library's
 * reading).  All arithmetic is IEEE double, summed in ascending key order.
 *
 * Inputs are read in their storage type (fp32, bf16 bit patterns, or fp64)
 * and widened exactly to double, so the oracle sees the very values the GPU
 * kernel sees.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

typedef struct {
  const void *q, *k, *v;
  int dtype;
  int64_t H, S, D;
  int causal;
  double scale;
  const int64_t *bh_idx;
  int64_t n_bh;
  const int64_t *row_idx;
  int64_t n_rows;
  double *o, *lse;
  int64_t item_begin, item_end; /* items are (bh, row) pairs, row-major over the sample lists */
  int64_t materialised;         /* score + probability elements this worker materialised */
  int status;
} job_t;

static double load_elem(const void *base, int dtype, int64_t idx) {
  switch (dtype) {
    case ORACLE_F32:
      return (double)((const float *)base)[idx];
    case ORACLE_BF16: {
      uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
      float f;
      memcpy(&f, &bits, sizeof f);
      return (double)f;
    }
    default:
      return ((const double *)base)[idx];
  }
}

static void *worker(void *arg) {
  job_t *j = (job_t *)arg;
  const int64_t S = j->S, D = j->D;
  double *scores = (double *)malloc(sizeof(double) * (size_t)S);
  double *probs = (double *)malloc(sizeof(double) * (size_t)S);
  double *qrow = (double *)malloc(sizeof(double) * (size_t)D);
  if (!scores || !probs || !qrow) {
    j->status = -2;
    free(scores); free(probs); free(qrow);
    return NULL;
  }
  for (int64_t it = j->item_begin; it < j->item_end; ++it) {
    const int64_t sb = it / j->n_rows, sr = it % j->n_rows;
    const int64_t bh = j->bh_idx ? j->bh_idx[sb] : sb;
    const int64_t i = j->row_idx ? j->row_idx[sr] : sr;
    const int64_t head = bh * S * D;
    const int64_t limit = j->causal ? i + 1 : S;
    for (int64_t c = 0; c < D; ++c) qrow[c] = load_elem(j->q, j->dtype, head + i * D + c);

    /* 1. the score row, materialised */
    for (int64_t kj = 0; kj < limit; ++kj) {
      double dot = 0.0;
      for (int64_t c = 0; c < D; ++c) dot += qrow[c] * load_elem(j->k, j->dtype, head + kj * D + c);
      scores[kj] = dot * j->scale;
    }
    /* 2. softmax with the row maximum subtracted, materialised */
    double m = scores[0];
    for (int64_t kj = 1; kj < limit; ++kj) m = scores[kj] > m ? scores[kj] : m;
    double denom = 0.0;
    for (int64_t kj = 0; kj < limit; ++kj) {
      probs[kj] = exp(scores[kj] - m);
      denom += probs[kj];
    }
    for (int64_t kj = 0; kj < limit; ++kj) probs[kj] = probs[kj] / denom;
    /* 3. the output row P V */
    double *orow = j->o + (sb * j->n_rows + sr) * D;
    for (int64_t c = 0; c < D; ++c) orow[c] = 0.0;
    for (int64_t kj = 0; kj < limit; ++kj) {
      const double p = probs[kj];
      for (int64_t c = 0; c < D; ++c) orow[c] += p * load_elem(j->v, j->dtype, head + kj * D + c);
    }
    if (j->lse) j->lse[sb * j->n_rows + sr] = m + log(denom);
    j->materialised += 2 * limit;
  }
  free(scores); free(probs); free(qrow);
  return NULL;
}

/*
 * Returns 0 on success, -1 for an invalid argument, -2 when memory or a
 * thread could not be obtained.  o is [n_bh][n_rows][D], lse [n_bh][n_rows]
 * (may be NULL).  NULL index lists select every head / every row.
 * *materialised (may be NULL) receives the number of score plus probability
 * elements that were materialised.
 */
int oracle_attention_dense(const void *q, const void *k, const void *v, int dtype, int64_t B,
                           int64_t H, int64_t S, int64_t D, int causal, double scale,
                           const int64_t *bh_idx, int64_t n_bh, const int64_t *row_idx,
                           int64_t n_rows, double *o, double *lse, int n_threads,
                           int64_t *materialised) {
  if (!q || !k || !v || !o || B < 1 || H < 1 || S < 1 || D < 1) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
  if (!bh_idx) n_bh = B * H;
  if (!row_idx) n_rows = S;
  if (n_bh < 1 || n_rows < 1) return -1;
  for (int64_t a = 0; bh_idx && a < n_bh; ++a)
    if (bh_idx[a] < 0 || bh_idx[a] >= B * H) return -1;
  for (int64_t a = 0; row_idx && a < n_rows; ++a)
    if (row_idx[a] < 0 || row_idx[a] >= S) return -1;

  const int64_t items = n_bh * n_rows;
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if ((int64_t)n_threads > items) n_threads = (int)items;
  job_t *jobs = (job_t *)calloc((size_t)n_threads, sizeof(job_t));
  pthread_t *tids = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
  char *created = (char *)calloc((size_t)n_threads, 1);
  if (!jobs || !tids || !created) {
    free(jobs); free(tids); free(created);
    return -2;
  }
  int status = 0;
  for (int t = 0; t < n_threads; ++t) {
    job_t *j = &jobs[t];
    j->q = q; j->k = k; j->v = v; j->dtype = dtype;
    j->H = H; j->S = S; j->D = D; j->causal = causal; j->scale = scale;
    j->bh_idx = bh_idx; j->n_bh = n_bh; j->row_idx = row_idx; j->n_rows = n_rows;
    j->o = o; j->lse = lse;
    j->item_begin = items * t / n_threads;
    j->item_end = items * (t + 1) / n_threads;
    if (t == n_threads - 1) {
      worker(j); /* the calling thread takes the last share */
    } else if (pthread_create(&tids[t], NULL, worker, j) == 0) {
      created[t] = 1;
    } else {
      worker(j);
    }
  }
  int64_t total = 0;
  for (int t = 0; t < n_threads; ++t)
    if (created[t]) pthread_join(tids[t], NULL);
  for (int t = 0; t < n_threads; ++t) {
    total += jobs[t].materialised;
    if (jobs[t].status) status = jobs[t].status;
  }
  if (materialised) *materialised = total;
  free(jobs); free(tids); free(created);
  return status;
}
