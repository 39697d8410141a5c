/*
 * MaxSim oracle: a plain, slow, float64 CPU implementation of what the GPU
 * library computes. TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the CPU-baseline leg of the benchmark may call it; the GPU library never
 * does. It shares no source with the GPU path.
 *
 * Definition (TileMaxSim deep reading, section 1; Flash-MaxSim abstract;
 * Flash-MaxSim page, axiom ledger): for a query of q_len tokens q_i and a
 * document of len_b tokens d_j,
 *
 *     score_b = sum_{i < q_len}  max_{j < len_b}  <q_i, d_j>
 *
 * computed on the stored values (raw inner product, no normalisation; the
 * inputs are already unit-norm). Every stored element is decoded exactly to
 * double; for bf16 / fp16 inputs every product is exact in double and the
 * 53-bit sums make the result exact up to the final rounding in practice.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - padding / tokens past a document's length are excluded from the max
 *    (max over the valid tokens only);
 *  - an empty document has max over nothing = -inf, so its score is -inf;
 *  - INT8 (Flash-MaxSim abstract: INT8xINT8 scoring; per-token symmetric
 *    scales): dot_ij is the exact integer dot product, the scaled similarity
 *    is v_ij = fl32( fl32(dot_ij) * fl32(s_qi * s_dj) ) in IEEE fp32 with
 *    round-to-nearest-even and no contraction, the per-token maximum is taken
 *    over v_ij with ties going to the lowest j, and score = sum_i m_i in double;
 *  - PQ (TileMaxSim deep reading, section 2 item (3)): per-query tables
 *    T[i][m][k] = <q_i[sub-vector m], C[m][k]>, a document token's similarity
 *    is the sum over subspaces of table entries picked by its codes,
 *    s_ij = sum_m T[i][m][c_jm], then max over j and sum over i as above.
 *    Sub-vector m covers dimensions [m*dsub, (m+1)*dsub).
 *  - per-token maxima and argmax (Flash-MaxSim abstract and the Flash-MaxSim
 *    page: the backward pass reuses the argmax locations of the forward): the
 *    argmax of query token i in document b is the lowest j reaching the maximum;
 *  - gradients (Flash-MaxSim abstract: training backward pass): with upstream
 *    gradient g_b of score_b and j*(b,i) the argmax, the score is linear in Q and
 *    D away from ties, so
 *        dQ[i]           = sum_b g_b * d_{b, j*(b,i)}
 *        dD[b, j]        = g_b * sum_{i : j*(b,i) = j} q_i   (zero if no i chose j)
 *    Documents without tokens (argmax -1) contribute nothing.
 *
 * Documents are independent, so they are split across threads; each
 * document's arithmetic is the same whatever thread runs it.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BF16 0
#define OR_FP16 1
#define OR_FP32 2

/* ---- exact decoding of stored elements ---- */

static double decode_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16; /* bf16 is the top half of an fp32 */
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double decode_fp16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exp = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (exp == 0)
    v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
  else if (exp == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + man), exp - 25); /* (1 + man/1024) * 2^(exp-15) */
  return sign ? -v : v;
}

static double decode(const void *base, int dtype, int64_t idx) {
  switch (dtype) {
  case OR_BF16: return decode_bf16(((const uint16_t *)base)[idx]);
  case OR_FP16: return decode_fp16(((const uint16_t *)base)[idx]);
  default: return (double)((const float *)base)[idx];
  }
}

/* ---- threading helper: run fn(ctx, b) for b in [0, n) over nthreads ---- */

typedef void (*doc_fn)(void *ctx, int64_t b);
typedef struct {
  doc_fn fn;
  void *ctx;
  int64_t b0, b1;
} range_job;

static void *range_worker(void *a) {
  range_job *j = (range_job *)a;
  for (int64_t b = j->b0; b < j->b1; b++) j->fn(j->ctx, b);
  return NULL;
}

static void for_each_doc(int64_t n, int nthreads, doc_fn fn, void *ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  pthread_t th[256];
  range_job jobs[256];
  for (int t = 0; t < nthreads; t++) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].b0 = n * t / nthreads;
    jobs[t].b1 = n * (t + 1) / nthreads;
    if (t > 0) pthread_create(&th[t], NULL, range_worker, &jobs[t]);
  }
  range_worker(&jobs[0]);
  for (int t = 1; t < nthreads; t++) pthread_join(th[t], NULL);
}

/* ---- dense MaxSim (bf16 / fp16 / fp32 storage) ---- */

typedef struct {
  const double *q; /* decoded query [q_len][d] */
  int q_len, d, dtype;
  const void *D;
  const int64_t *offsets;  /* CSR: token range of doc b; NULL for the fixed layout */
  int nd;                  /* fixed layout: tokens per doc slot */
  const int32_t *doc_lens; /* fixed layout: valid tokens per doc (NULL = nd) */
  double *out;
  double *tok_max;         /* [n_docs][q_len] per-token maxima, nullable */
  int32_t *tok_arg;        /* [n_docs][q_len] lowest index reaching the maximum, nullable */
} dense_ctx;

static void dense_doc(void *vctx, int64_t b) {
  const dense_ctx *c = (const dense_ctx *)vctx;
  int64_t first;
  int64_t len;
  if (c->offsets) {
    first = c->offsets[b];
    len = c->offsets[b + 1] - c->offsets[b];
  } else {
    first = b * (int64_t)c->nd;
    len = c->nd;
    if (c->doc_lens) {
      len = c->doc_lens[b];
      if (len < 0) len = 0;
      if (len > c->nd) len = c->nd;
    }
  }
  double score = 0.0;
  for (int i = 0; i < c->q_len; i++) {
    double m = -INFINITY;
    int32_t arg = -1;
    for (int64_t j = 0; j < len; j++) {
      double s = 0.0;
      for (int k = 0; k < c->d; k++)
        s += c->q[(int64_t)i * c->d + k] * decode(c->D, c->dtype, (first + j) * c->d + k);
      if (s > m) { /* strict: the first maximum is kept */
        m = s;
        arg = (int32_t)j;
      }
    }
    if (c->tok_max) c->tok_max[b * c->q_len + i] = m;
    if (c->tok_arg) c->tok_arg[b * c->q_len + i] = arg;
    score += m;
  }
  c->out[b] = score;
}

static double *decode_query(const void *Q, int q_len, int d, int dtype) {
  double *q = (double *)malloc(sizeof(double) * (size_t)q_len * (size_t)d);
  for (int64_t e = 0; e < (int64_t)q_len * d; e++) q[e] = decode(Q, dtype, e);
  return q;
}

/* CSR documents: tokens D[offsets[n_docs]][d]; doc b is rows [offsets[b], offsets[b+1]). */
int oracle_maxsim_csr(const void *Q, int q_len, const void *D, const int64_t *offsets,
                      int64_t n_docs, int d, int dtype, double *out, int nthreads) {
  if (!Q || !D || !offsets || !out || q_len < 0 || d <= 0 || n_docs < 0) return -1;
  if (dtype < OR_BF16 || dtype > OR_FP32) return -1;
  dense_ctx c = {decode_query(Q, q_len, d, dtype), q_len, d, dtype, D, offsets, 0, NULL, out,
                 NULL, NULL};
  for_each_doc(n_docs, nthreads, dense_doc, &c);
  free((void *)c.q);
  return 0;
}

/* Fixed layout: D[n_docs][nd][d]; doc_lens (nullable) masks tokens j >= doc_lens[b]. */
int oracle_maxsim_fixed(const void *Q, int q_len, const void *D, int64_t n_docs, int nd,
                        const int32_t *doc_lens, int d, int dtype, double *out, int nthreads) {
  if (!Q || !D || !out || q_len < 0 || d <= 0 || n_docs < 0 || nd < 0) return -1;
  if (dtype < OR_BF16 || dtype > OR_FP32) return -1;
  dense_ctx c = {decode_query(Q, q_len, d, dtype), q_len, d, dtype, D, NULL, nd, doc_lens, out,
                 NULL, NULL};
  for_each_doc(n_docs, nthreads, dense_doc, &c);
  free((void *)c.q);
  return 0;
}

/* Scores with per-token maxima and argmax. offsets nullable: fixed layout D[n_docs][nd][d]. */
int oracle_maxsim_argmax(const void *Q, int q_len, const void *D, const int64_t *offsets,
                         int64_t n_docs, int nd, int d, int dtype, double *out, double *tok_max,
                         int32_t *tok_arg, int nthreads) {
  if (!Q || !D || !out || !tok_max || !tok_arg || q_len < 0 || d <= 0 || n_docs < 0) return -1;
  if (!offsets && nd < 0) return -1;
  if (dtype < OR_BF16 || dtype > OR_FP32) return -1;
  dense_ctx c = {decode_query(Q, q_len, d, dtype), q_len, d, dtype, D, offsets, nd, NULL, out,
                 tok_max, tok_arg};
  for_each_doc(n_docs, nthreads, dense_doc, &c);
  free((void *)c.q);
  return 0;
}

/* Gradients of sum_b grad[b] * score_b given the argmax tok_arg[n_docs][q_len]:
 * dQ[q_len][d] and dD[n_tokens][d] (n_tokens = offsets[n_docs], or n_docs * nd), in double;
 * either output may be NULL (not computed).
 * An argmax outside [0, len_b) (the -1 of an empty document) contributes nothing. */
int oracle_maxsim_backward(const void *Q, int q_len, const void *D, const int64_t *offsets,
                           int64_t n_docs, int nd, int d, int dtype, const int32_t *tok_arg,
                           const float *grad, double *dQ, double *dD) {
  if (!Q || !D || !tok_arg || !grad || q_len < 0 || d <= 0 || n_docs < 0) return -1;
  if (!offsets && nd < 0) return -1;
  if (dtype < OR_BF16 || dtype > OR_FP32) return -1;
  double *q = decode_query(Q, q_len, d, dtype);
  const int64_t n_tokens = offsets ? offsets[n_docs] : n_docs * (int64_t)nd;
  if (dQ) memset(dQ, 0, sizeof(double) * (size_t)q_len * (size_t)d);
  if (dD) memset(dD, 0, sizeof(double) * (size_t)n_tokens * (size_t)d);
  for (int64_t b = 0; b < n_docs; b++) {
    const int64_t first = offsets ? offsets[b] : b * (int64_t)nd;
    const int64_t len = offsets ? offsets[b + 1] - offsets[b] : nd;
    const double g = (double)grad[b];
    for (int i = 0; i < q_len; i++) {
      const int64_t j = tok_arg[b * q_len + i];
      if (j < 0 || j >= len) continue;
      for (int k = 0; k < d; k++) {
        if (dQ) dQ[(int64_t)i * d + k] += g * decode(D, dtype, (first + j) * d + k);
        if (dD) dD[(first + j) * d + k] += g * q[(int64_t)i * d + k];
      }
    }
  }
  free(q);
  return 0;
}

/* ---- INT8 x INT8 with per-token fp32 scales ---- */

typedef struct {
  const int8_t *Q;
  const float *qs;
  int q_len, d, nd;
  const int8_t *D;
  const float *ds;
  const int64_t *offsets;
  double *out;
  float *tok_max;    /* [n_docs][q_len], nullable */
  int32_t *tok_arg;  /* [n_docs][q_len], nullable */
} i8_ctx;

static void i8_doc(void *vctx, int64_t b) {
  const i8_ctx *c = (const i8_ctx *)vctx;
  int64_t first = c->offsets ? c->offsets[b] : b * (int64_t)c->nd;
  int64_t len = c->offsets ? c->offsets[b + 1] - c->offsets[b] : c->nd;
  double score = 0.0;
  for (int i = 0; i < c->q_len; i++) {
    float m = -INFINITY;
    int32_t arg = -1;
    for (int64_t j = 0; j < len; j++) {
      int64_t dot = 0;
      for (int k = 0; k < c->d; k++)
        dot += (int64_t)c->Q[(int64_t)i * c->d + k] * (int64_t)c->D[(first + j) * c->d + k];
      volatile float scale = c->qs[i] * c->ds[first + j]; /* one fp32 rounding */
      volatile float v = (float)dot * scale;               /* one fp32 rounding */
      if (v > m) { /* strict: ties keep the lowest j */
        m = v;
        arg = (int32_t)j;
      }
    }
    if (c->tok_max) c->tok_max[b * c->q_len + i] = m;
    if (c->tok_arg) c->tok_arg[b * c->q_len + i] = arg;
    score += (double)m;
  }
  c->out[b] = score;
}

/* offsets nullable: then the layout is fixed, D[n_docs][nd][d], d_scale[n_docs][nd]. */
int oracle_maxsim_i8(const int8_t *Q, const float *q_scale, int q_len, const int8_t *D,
                     const float *d_scale, const int64_t *offsets, int64_t n_docs, int nd, int d,
                     double *out, float *tok_max, int32_t *tok_arg, int nthreads) {
  if (!Q || !q_scale || !D || !d_scale || !out || q_len < 0 || d <= 0 || n_docs < 0) return -1;
  if (!offsets && nd < 0) return -1;
  i8_ctx c = {Q, q_scale, q_len, d, nd, D, d_scale, offsets, out, tok_max, tok_arg};
  for_each_doc(n_docs, nthreads, i8_doc, &c);
  return 0;
}

/* ---- product quantisation ---- */

/* T[i][m][k] = sum_{t < dsub} q_i[m*dsub + t] * C[m][k][t], in double. */
int oracle_pq_tables(const void *Q, int q_len, int dtype, const float *C, int M, int K, int dsub,
                     double *T) {
  if (!Q || !C || !T || q_len < 0 || M <= 0 || K <= 0 || dsub <= 0) return -1;
  if (dtype < OR_BF16 || dtype > OR_FP32) return -1;
  int d = M * dsub;
  for (int i = 0; i < q_len; i++)
    for (int m = 0; m < M; m++)
      for (int k = 0; k < K; k++) {
        double s = 0.0;
        for (int t = 0; t < dsub; t++)
          s += decode(Q, dtype, (int64_t)i * d + (int64_t)m * dsub + t) *
               (double)C[((int64_t)m * K + k) * dsub + t];
        T[((int64_t)i * M + m) * K + k] = s;
      }
  return 0;
}

typedef struct {
  const double *T;
  int q_len, M, K, nd;
  const uint8_t *codes;
  const int64_t *offsets;
  double *out;
} pq_ctx;

static void pq_doc(void *vctx, int64_t b) {
  const pq_ctx *c = (const pq_ctx *)vctx;
  int64_t first = c->offsets ? c->offsets[b] : b * (int64_t)c->nd;
  int64_t len = c->offsets ? c->offsets[b + 1] - c->offsets[b] : c->nd;
  double score = 0.0;
  for (int i = 0; i < c->q_len; i++) {
    double mx = -INFINITY;
    for (int64_t j = 0; j < len; j++) {
      double s = 0.0;
      for (int m = 0; m < c->M; m++) {
        int code = c->codes[(first + j) * c->M + m];
        s += c->T[((int64_t)i * c->M + m) * c->K + code];
      }
      if (s > mx) mx = s;
    }
    score += mx;
  }
  c->out[b] = score;
}

/* codes[tokens][M] uint8; offsets nullable => fixed layout of nd tokens per doc. */
int oracle_maxsim_pq(const double *T, int q_len, int M, int K, const uint8_t *codes,
                     const int64_t *offsets, int64_t n_docs, int nd, double *out, int nthreads) {
  if (!T || !codes || !out || q_len < 0 || M <= 0 || K <= 0 || n_docs < 0) return -1;
  if (!offsets && nd < 0) return -1;
  pq_ctx c = {T, q_len, M, K, nd, codes, offsets, out};
  for_each_doc(n_docs, nthreads, pq_doc, &c);
  return 0;
}
