/*
 * decode_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct fp64 CPU reference for single-token decode
 * attention. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library; the product path never does.
 *
 * What it computes is the plain definition of attention for one query token,
 *     out[b,h,:] = sum_j softmax_j(scale * q[b,h,:] . k[bk,hk,j,:]) * v[bk,hk,j,:]
 * written out in fp64 over bfloat16 inputs:
 *   - fuel-dispatch page "DecodeFlashSpec": q is [B, Hq, Sq, D]; k and v are the
 *     capacity KV buffers [B, Hkv, capacity, D]; softmax_scale is an f32; the
 *     query attends the live prefix [0, k_len) (field k_len); with Sq = 1 the
 *     causal flag changes nothing (field causal). The decomposed arm is named
 *     there as the oracle (field decomposed_out): this file plays that role.
 *   - metrale page "AttnV41", decode_fixed_topk and decode_prep: in the sparse
 *     variant each token attends the rows named by its padded selection; a -1
 *     pad contributes to neither the softmax sum nor the weighted sum of values.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *   - query head h reads KV head h / (Hq / Hkv) (contiguous GQA groups);
 *   - the scale multiplies the fp64 score; it is never folded into q;
 *   - any negative selection entry is a pad; an entry >= k_len is a caller
 *     error, reported here with a nonzero return code;
 *   - duplicate entries count with multiplicity (list semantics);
 *   - a row whose selection holds no valid entry has output 0;
 *   - for the sparse call, kv_batch == 1 means every token reads the one
 *     shared set of rows; kv_batch == B means token b reads set b.
 *
 * No blocking, no fusion, no online rescaling: scores for the whole key list
 * are formed first, then their maximum, then the weights, then the sums, in
 * ascending key-list order and ascending d. Work is spread over threads by
 * whole (b, h) rows, which does not change any row's arithmetic.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Exact widening of a bfloat16 bit pattern: the top half of an IEEE binary32. */
static double bf16_to_double(uint16_t u) {
  uint32_t w = (uint32_t)u << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

typedef struct {
  const uint16_t *q, *k, *v;
  const int32_t *sel; /* NULL for the dense call */
  int32_t topk;
  double *out;
  int32_t B, Hq, Hkv, D, kv_batch;
  int64_t capacity, k_len;
  double scale;
  const int64_t *rows; /* flattened b*Hq + h; NULL = all rows in order */
  int64_t nrows;
  int64_t next;        /* next row index to take (guarded by lock) */
  pthread_mutex_t lock;
  int error;
} job_t;

/* One (b, h) row. Returns 0, or 1 on an out-of-range selection entry. */
static int attend_row(const job_t *J, int64_t row, double *out, double *scores,
                      int64_t *keys) {
  const int32_t b = (int32_t)(row / J->Hq), h = (int32_t)(row % J->Hq);
  const int32_t G = J->Hq / J->Hkv;
  const int32_t hk = h / G;
  const int32_t D = J->D;
  const int32_t bk = J->sel ? (J->kv_batch == 1 ? 0 : b) : b;

  /* The key list: [0, k_len) for the dense call, or the valid entries of the
   * selection in list order for the sparse call. */
  int64_t n = 0;
  if (!J->sel) {
    for (int64_t j = 0; j < J->k_len; ++j) keys[n++] = j;
  } else {
    for (int32_t t = 0; t < J->topk; ++t) {
      int32_t r = J->sel[(int64_t)b * J->topk + t];
      if (r < 0) continue;             /* a pad: contributes nothing */
      if ((int64_t)r >= J->k_len) return 1;
      keys[n++] = r;
    }
  }
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (n == 0) return 0;

  const uint16_t *qrow = J->q + ((int64_t)b * J->Hq + h) * D;
  const uint16_t *kbase = J->k + ((int64_t)bk * J->Hkv + hk) * J->capacity * D;
  const uint16_t *vbase = J->v + ((int64_t)bk * J->Hkv + hk) * J->capacity * D;

  /* Scores s_j = scale * (q . k_j). */
  for (int64_t i = 0; i < n; ++i) {
    const uint16_t *krow = kbase + keys[i] * D;
    double dot = 0.0;
    for (int32_t d = 0; d < D; ++d) dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
    scores[i] = J->scale * dot;
  }
  /* Softmax with the maximum subtracted: w_j = exp(s_j - m), Z = sum w_j. */
  double m = scores[0];
  for (int64_t i = 1; i < n; ++i)
    if (scores[i] > m) m = scores[i];
  double Z = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    scores[i] = exp(scores[i] - m);
    Z += scores[i];
  }
  /* out_d = (sum_j w_j v_jd) / Z. */
  for (int64_t i = 0; i < n; ++i) {
    const uint16_t *vrow = vbase + keys[i] * D;
    for (int32_t d = 0; d < D; ++d) out[d] += scores[i] * bf16_to_double(vrow[d]);
  }
  for (int32_t d = 0; d < D; ++d) out[d] /= Z;
  return 0;
}

static void *worker(void *arg) {
  job_t *J = (job_t *)arg;
  int64_t cap = J->sel ? J->topk : J->k_len;
  if (cap < 1) cap = 1;
  double *scores = (double *)malloc(sizeof(double) * (size_t)cap);
  int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
  if (!scores || !keys) {
    pthread_mutex_lock(&J->lock);
    J->error = 3;
    pthread_mutex_unlock(&J->lock);
    free(scores);
    free(keys);
    return NULL;
  }
  for (;;) {
    pthread_mutex_lock(&J->lock);
    int64_t i = J->next++;
    int err = J->error;
    pthread_mutex_unlock(&J->lock);
    if (i >= J->nrows || err) break;
    int64_t row = J->rows ? J->rows[i] : i;
    if (attend_row(J, row, J->out + i * J->D, scores, keys)) {
      pthread_mutex_lock(&J->lock);
      J->error = 2;
      pthread_mutex_unlock(&J->lock);
    }
  }
  free(scores);
  free(keys);
  return NULL;
}

static int run(job_t *J, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 1024) nthreads = 1024;
  pthread_mutex_init(&J->lock, NULL);
  J->next = 0;
  J->error = 0;
  pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!tid) return 3;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    if (pthread_create(&tid[t], NULL, worker, J) != 0) break;
    ++started;
  }
  if (started == 0) worker(J);
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
  free(tid);
  pthread_mutex_destroy(&J->lock);
  return J->error;
}

static int check_shape(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t capacity,
                       int64_t k_len) {
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv != 0) return 1;
  if (k_len < 1 || k_len > capacity) return 1;
  return 0;
}

/* Dense: q [B,Hq,1,D], k/v [B,Hkv,capacity,D] (bf16 bits); out [nrows, D] fp64
 * for the listed flattened rows b*Hq+h (all rows when rows == NULL).
 * Returns 0 on success, 1 on bad shapes, 3 on allocation failure. */
int oracle_dense(const uint16_t *q, const uint16_t *k, const uint16_t *v, double *out,
                 int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t capacity,
                 int64_t k_len, float scale, const int64_t *rows, int64_t nrows,
                 int nthreads) {
  if (check_shape(B, Hq, Hkv, D, capacity, k_len)) return 1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.sel = NULL; J.topk = 0; J.out = out;
  J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.kv_batch = B;
  J.capacity = capacity; J.k_len = k_len; J.scale = (double)scale;
  J.rows = rows; J.nrows = rows ? nrows : (int64_t)B * Hq;
  return run(&J, nthreads);
}

/* Sparse: q [B,Hq,1,D], k/v [kv_batch,Hkv,capacity,D], sel [B,topk] int32;
 * rows usable by the selection are [0, k_len). Same return codes as dense,
 * plus 2 when a selection entry is >= k_len. */
int oracle_sparse(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const int32_t *sel, int32_t topk, double *out, int32_t B, int32_t Hq,
                  int32_t Hkv, int32_t D, int32_t kv_batch, int64_t capacity, int64_t k_len,
                  float scale, const int64_t *rows, int64_t nrows, int nthreads) {
  if (check_shape(B, Hq, Hkv, D, capacity, k_len)) return 1;
  if (topk < 0 || !(kv_batch == 1 || kv_batch == B)) return 1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.sel = sel; J.topk = topk; J.out = out;
  J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.kv_batch = kv_batch;
  J.capacity = capacity; J.k_len = k_len; J.scale = (double)scale;
  J.rows = rows; J.nrows = rows ? nrows : (int64_t)B * Hq;
  return run(&J, nthreads);
}
