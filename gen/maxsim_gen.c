/*
 * Seeded synthetic inputs for late-interaction MaxSim scoring.
 *
 * This file produces inputs only. It holds none of the scoring arithmetic:
 * no dot products, no maxima, no sums over query tokens. Both the CPU oracle
 * and the GPU library read the bytes written here.
 *
 * Random numbers are counter-based, so any token of any document can be
 * regenerated on its own, and the output does not depend on the number of
 * threads:
 *   - SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): the i-th output of a generator seeded with
 *     `key` is mix(key + (i + 1) * GOLDEN).
 *   - uniform in (0, 1]: ((x >> 11) + 1) * 2^-53.
 *   - normal: Box & Muller (1958), from the uniform pair (2p, 2p + 1).
 *
 * Workload shapes follow the pages' benchmark descriptions: ColBERTv2-shaped
 * unit-norm token embeddings (TileMaxSim deep reading, section 2, test
 * environment: d=128, Nq=32, Nd in {64,128,256}), ColPali-shaped long
 * sequences (Flash-MaxSim, Figure 2: Lq=Ld=1024), lognormal document lengths
 * for a variable-length corpus (TileMaxSim deep reading, section 5: padding of
 * variable-length corpora), INT8 per-token symmetric quantisation and PQ codes
 * (TileMaxSim deep reading, section 2 item (3)).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GEN_BF16 0
#define GEN_FP16 1
#define GEN_FP32 2
#define GEN_F64 3
#define GEN_I8 4

static const uint64_t GOLDEN = 0x9e3779b97f4a7c15ULL;

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

/* Key of the (seed, stream) generator: two SplitMix64 steps. */
uint64_t gen_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN) + (stream + 1) * GOLDEN);
}

/* i-th 64-bit output of the generator with this key. */
uint64_t gen_u64(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

static double u01(uint64_t x) { return ((double)(x >> 11) + 1.0) * 0x1.0p-53; }

/* n-th standard normal of the stream (Box-Muller over the pair n/2). */
double gen_normal(uint64_t key, uint64_t n) {
  uint64_t p = n >> 1;
  double u1 = u01(gen_u64(key, 2 * p));
  double u2 = u01(gen_u64(key, 2 * p + 1));
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (n & 1) ? r * sin(a) : r * cos(a);
}

/* ---- storage rounding: double -> fp32 (RNE) -> bf16 / fp16 (RNE) ---- */

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* NaN */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static uint16_t f32_to_f16_rne(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7fffffffu;
  if (ax > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);  /* NaN */
  if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u); /* >= 65520 -> inf */
  if (ax < 0x38800000u) {
    /* below 2^-14: fp16 subnormal (or zero), units of 2^-24, round half even */
    float a;
    memcpy(&a, &ax, 4);
    double m = nearbyint((double)a * 16777216.0);
    return (uint16_t)(sign | (uint32_t)m); /* m == 1024 is the smallest normal */
  }
  uint32_t h = ((((ax >> 23) - 127u + 15u) << 10) | ((ax & 0x7fffffu) >> 13));
  uint32_t rem = ax & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
  return (uint16_t)(sign | h);
}

/* Store one double token row of length d in the requested format. */
static void store_row(const double *x, int d, int dtype, void *out, int64_t row, float *scale) {
  switch (dtype) {
  case GEN_BF16: {
    uint16_t *o = (uint16_t *)out + row * d;
    for (int e = 0; e < d; e++) o[e] = f32_to_bf16_rne((float)x[e]);
    break;
  }
  case GEN_FP16: {
    uint16_t *o = (uint16_t *)out + row * d;
    for (int e = 0; e < d; e++) o[e] = f32_to_f16_rne((float)x[e]);
    break;
  }
  case GEN_FP32: {
    float *o = (float *)out + row * d;
    for (int e = 0; e < d; e++) o[e] = (float)x[e];
    break;
  }
  case GEN_F64: {
    double *o = (double *)out + row * d;
    for (int e = 0; e < d; e++) o[e] = x[e];
    break;
  }
  case GEN_I8: {
    /* symmetric per-token quantisation: s = fl32(max|x| / 127),
       q = clamp(round_half_even(x / s), -127, 127); a zero token gives s = 0, q = 0 */
    int8_t *o = (int8_t *)out + row * d;
    double amax = 0.0;
    for (int e = 0; e < d; e++) amax = fmax(amax, fabs(x[e]));
    float s = (float)(amax / 127.0);
    for (int e = 0; e < d; e++) {
      double q = (s > 0.0f) ? nearbyint(x[e] / (double)s) : 0.0;
      if (q > 127.0) q = 127.0;
      if (q < -127.0) q = -127.0;
      o[e] = (int8_t)q;
    }
    scale[row] = s;
    break;
  }
  }
}

static void normalise(double *x, int d) {
  double ss = 0.0;
  for (int e = 0; e < d; e++) ss += x[e] * x[e];
  double inv = 1.0 / sqrt(ss);
  for (int e = 0; e < d; e++) x[e] *= inv;
}

/* Unit-norm Gaussian token `row` of the stream, in double. */
void gen_unit_token(uint64_t seed, uint64_t stream, int64_t row, int d, double *x) {
  uint64_t key = gen_key(seed, stream);
  for (int e = 0; e < d; e++) x[e] = gen_normal(key, (uint64_t)row * (uint64_t)d + (uint64_t)e);
  normalise(x, d);
}

/* ---- threaded bulk generation ---- */

typedef struct {
  uint64_t seed, stream;
  int64_t row0, r_begin, r_end;
  int d, dtype;
  void *out;
  float *scale;
} tok_job;

static void *tok_worker(void *arg) {
  tok_job *j = (tok_job *)arg;
  double *x = (double *)malloc(sizeof(double) * (size_t)j->d);
  for (int64_t r = j->r_begin; r < j->r_end; r++) {
    gen_unit_token(j->seed, j->stream, j->row0 + r, j->d, x);
    store_row(x, j->d, j->dtype, j->out, r, j->scale);
  }
  free(x);
  return NULL;
}

/*
 * Rows [row0, row0 + nrows) of a unit-norm Gaussian token stream, stored as
 * dtype into out[nrows][d] (row r of out is stream row row0 + r). For GEN_I8,
 * scale[nrows] receives the per-token fp32 scale.
 */
int gen_tokens(uint64_t seed, uint64_t stream, int64_t row0, int64_t nrows, int d, int dtype,
               void *out, float *scale, int nthreads) {
  if (d <= 0 || nrows < 0 || !out || dtype < 0 || dtype > GEN_I8) return -1;
  if (dtype == GEN_I8 && !scale) return -1;
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > nrows / 256 + 1) nthreads = (int)(nrows / 256 + 1);
  pthread_t th[256];
  tok_job jobs[256];
  if (nthreads > 256) nthreads = 256;
  for (int t = 0; t < nthreads; t++) {
    tok_job *j = &jobs[t];
    j->seed = seed;
    j->stream = stream;
    j->row0 = row0;
    j->r_begin = nrows * t / nthreads;
    j->r_end = nrows * (t + 1) / nthreads;
    j->d = d;
    j->dtype = dtype;
    j->out = out;
    j->scale = scale;
    if (t > 0) pthread_create(&th[t], NULL, tok_worker, j);
  }
  tok_worker(&jobs[0]);
  for (int t = 1; t < nthreads; t++) pthread_join(th[t], NULL);
  return 0;
}

/*
 * Lognormal document lengths: L_b = clip(round(exp(ln(median) + sigma * z_b)), lo, hi),
 * z_b the b-th normal of the stream; round half away from zero.
 */
int gen_lengths(uint64_t seed, uint64_t stream, int64_t n_docs, double median, double sigma,
                int lo, int hi, int32_t *out) {
  if (!out || n_docs < 0 || lo < 0 || hi < lo || median <= 0.0) return -1;
  uint64_t key = gen_key(seed, stream);
  for (int64_t b = 0; b < n_docs; b++) {
    double v = round(exp(log(median) + sigma * gen_normal(key, (uint64_t)b)));
    if (v < lo) v = lo;
    if (v > hi) v = hi;
    out[b] = (int32_t)v;
  }
  return 0;
}

/* n distinct values in [0, range), drawn by rejection from the stream, in draw order. */
int gen_distinct(uint64_t seed, uint64_t stream, uint64_t salt, int n, int64_t range, int64_t *out) {
  if (!out || n < 0 || (int64_t)n > range) return -1;
  uint64_t key = gen_key(seed, stream);
  uint64_t i = salt << 32;
  for (int c = 0; c < n;) {
    int64_t v = (int64_t)(gen_u64(key, i++) % (uint64_t)range);
    int dup = 0;
    for (int k = 0; k < c; k++) dup |= (out[k] == v);
    if (!dup) out[c++] = v;
  }
  return 0;
}

/*
 * Plant the query into one document as a near-duplicate. For the planted
 * document `doc_id` of length len, min(nq, len) distinct positions p_i are drawn
 * (planting stream, salt doc_id + 1); token p_i becomes normalise(q_i + sigma * z),
 * with q_i the double unit-norm query token i (query stream row q_row0 + i) and
 * z fresh normals of the noise stream. The planted tokens are written, stored as
 * dtype, at rows p_i of doc_rows (the document's own token rows).
 */
int gen_plant_doc(uint64_t seed, uint64_t q_stream, int64_t q_row0, int nq, uint64_t plant_stream,
                  uint64_t noise_stream, int64_t doc_id, int len, int d, double sigma, int dtype,
                  void *doc_rows, float *doc_scale) {
  if (!doc_rows || nq <= 0 || len <= 0 || d <= 0) return -1;
  if (dtype == GEN_I8 && !doc_scale) return -1;
  int n = nq < len ? nq : len;
  int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
  int64_t *which = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
  double *x = (double *)malloc(sizeof(double) * (size_t)d);
  gen_distinct(seed, plant_stream, (uint64_t)doc_id + 1, n, len, pos);
  /* which query tokens are planted when len < nq: a seeded subset */
  if (n < nq)
    gen_distinct(seed, plant_stream, (uint64_t)doc_id + 1 + (1ull << 31), n, nq, which);
  else
    for (int i = 0; i < n; i++) which[i] = i;
  uint64_t nkey = gen_key(seed, noise_stream);
  for (int i = 0; i < n; i++) {
    gen_unit_token(seed, q_stream, q_row0 + which[i], d, x);
    for (int e = 0; e < d; e++)
      x[e] += sigma * gen_normal(nkey, ((uint64_t)doc_id * (uint64_t)nq + (uint64_t)which[i]) *
                                               (uint64_t)d + (uint64_t)e);
    normalise(x, d);
    store_row(x, d, dtype, doc_rows, pos[i], doc_scale);
  }
  free(pos);
  free(which);
  free(x);
  return 0;
}

/* PQ codebook C[M][K][dsub], each centroid a unit-norm Gaussian vector, fp32. */
int gen_codebook(uint64_t seed, uint64_t stream, int M, int K, int dsub, float *C) {
  if (!C || M <= 0 || K <= 0 || dsub <= 0) return -1;
  double *x = (double *)malloc(sizeof(double) * (size_t)dsub);
  for (int64_t r = 0; r < (int64_t)M * K; r++) {
    gen_unit_token(seed, stream, r, dsub, x);
    for (int t = 0; t < dsub; t++) C[r * dsub + t] = (float)x[t];
  }
  free(x);
  return 0;
}

/* Uniform PQ codes codes[n_tokens][M] in [0, K), K <= 256, from the stream. */
int gen_codes(uint64_t seed, uint64_t stream, int64_t row0, int64_t n_tokens, int M, int K,
              uint8_t *codes) {
  if (!codes || M <= 0 || K <= 0 || K > 256 || n_tokens < 0) return -1;
  uint64_t key = gen_key(seed, stream);
  for (int64_t r = 0; r < n_tokens; r++)
    for (int m = 0; m < M; m++)
      codes[r * M + m] =
          (uint8_t)(gen_u64(key, (uint64_t)(row0 + r) * (uint64_t)M + (uint64_t)m) % (uint64_t)K);
  return 0;
}

/*
 * PQ encoding of double token rows x[n][M*dsub]: code m of a token is the index
 * of the centroid C[m][k] nearest in squared L2 distance to the token's
 * sub-vector m (dimensions [m*dsub, (m+1)*dsub)); ties go to the lowest k.
 */
int gen_pq_encode(const double *x, int64_t n, int M, int K, int dsub, const float *C,
                  uint8_t *codes) {
  if (!x || !C || !codes || K > 256) return -1;
  for (int64_t r = 0; r < n; r++)
    for (int m = 0; m < M; m++) {
      const double *xs = x + r * (int64_t)M * dsub + (int64_t)m * dsub;
      double best = INFINITY;
      int arg = 0;
      for (int k = 0; k < K; k++) {
        const float *c = C + ((int64_t)m * K + k) * dsub;
        double dist = 0.0;
        for (int t = 0; t < dsub; t++) dist += (xs[t] - c[t]) * (xs[t] - c[t]);
        if (dist < best) {
          best = dist;
          arg = k;
        }
      }
      codes[r * M + m] = (uint8_t)arg;
    }
  return 0;
}

/*
 * Rows [row0, row0 + n) of a unit-norm Gaussian token stream (d = M * dsub), each
 * generated in double and encoded as gen_pq_encode does (nearest centroid of each
 * sub-vector, ties to the lowest k), over nthreads threads: PQ codes of a corpus
 * without holding its vectors.
 */
typedef struct {
  uint64_t seed, stream;
  int64_t row0, r_begin, r_end;
  int M, K, dsub;
  const float *C;
  uint8_t *codes;
} enc_job;

/* The same distances and choice as gen_pq_encode, laid out so that the loop over the
 * centroids is innermost (each centroid's sum still runs over t in increasing order). */
static void *enc_worker(void *arg) {
  enc_job *j = (enc_job *)arg;
  const int M = j->M, K = j->K, dsub = j->dsub, d = M * dsub;
  double *x = (double *)malloc(sizeof(double) * (size_t)d);
  double *dist = (double *)malloc(sizeof(double) * (size_t)K);
  double *ct = (double *)malloc(sizeof(double) * (size_t)M * dsub * K);  /* [m][t][k] */
  for (int m = 0; m < M; m++)
    for (int t = 0; t < dsub; t++)
      for (int k = 0; k < K; k++)
        ct[((size_t)m * dsub + t) * K + k] = (double)j->C[((size_t)m * K + k) * dsub + t];
  for (int64_t r = j->r_begin; r < j->r_end; r++) {
    gen_unit_token(j->seed, j->stream, j->row0 + r, d, x);
    for (int m = 0; m < M; m++) {
      for (int k = 0; k < K; k++) dist[k] = 0.0;
      for (int t = 0; t < dsub; t++) {
        const double xt = x[m * dsub + t];
        const double *c = ct + ((size_t)m * dsub + t) * K;
        for (int k = 0; k < K; k++) dist[k] += (xt - c[k]) * (xt - c[k]);
      }
      double best = INFINITY;
      int arg = 0;
      for (int k = 0; k < K; k++)
        if (dist[k] < best) {
          best = dist[k];
          arg = k;
        }
      j->codes[r * M + m] = (uint8_t)arg;
    }
  }
  free(ct);
  free(dist);
  free(x);
  return NULL;
}

int gen_encoded_codes(uint64_t seed, uint64_t stream, int64_t row0, int64_t n, int M, int K,
                      int dsub, const float *C, uint8_t *codes, int nthreads) {
  if (n < 0 || M < 1 || K < 1 || K > 256 || dsub < 1 || !C || !codes) return -1;
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > n / 64 + 1) nthreads = (int)(n / 64 + 1);
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  enc_job jobs[256];
  for (int t = 0; t < nthreads; t++) {
    enc_job *j = &jobs[t];
    j->seed = seed;
    j->stream = stream;
    j->row0 = row0;
    j->r_begin = n * t / nthreads;
    j->r_end = n * (t + 1) / nthreads;
    j->M = M;
    j->K = K;
    j->dsub = dsub;
    j->C = C;
    j->codes = codes;
    if (t > 0) pthread_create(&th[t], NULL, enc_worker, j);
  }
  enc_worker(&jobs[0]);
  for (int t = 1; t < nthreads; t++) pthread_join(th[t], NULL);
  return 0;
}

/* Storage rounding exposed for tests of the encoders. */
void gen_round_f32_to_bf16(const float *x, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = f32_to_bf16_rne(x[i]);
}
void gen_round_f32_to_f16(const float *x, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = f32_to_f16_rne(x[i]);
}
