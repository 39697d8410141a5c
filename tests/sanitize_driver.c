/*
 * Host-side sanitizer driver for the input generator and the CPU oracle.
 *
 * Built by tests/test_sanitizers.py together with gen/maxsim_gen.c and
 * oracle/maxsim_oracle.c under AddressSanitizer + UndefinedBehaviorSanitizer,
 * and again under ThreadSanitizer, then run as a child process. It calls every
 * exported function of both on small inputs that reach their edge cases (empty
 * documents, masked tokens, one-token documents, ragged CSR tails, several
 * threads, argmax outputs, null optional outputs), so an out-of-bounds access,
 * a use after free, undefined integer behaviour or a data race between the
 * threads that split the documents stops the run with a report.
 * Prints "sanitize driver: ok" when every call returned 0 and every score is a
 * number (or -inf for an empty document).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* generator (gen/maxsim_gen.c) */
int gen_tokens(uint64_t seed, uint64_t stream, int64_t row0, int64_t nrows, int d, int dtype,
               void *out, float *scale, int nthreads);
int gen_lengths(uint64_t seed, uint64_t stream, int64_t n_docs, double median, double sigma,
                int lo, int hi, int32_t *out);
int gen_distinct(uint64_t seed, uint64_t stream, uint64_t salt, int n, int64_t range, int64_t *out);
int gen_plant_doc(uint64_t seed, uint64_t q_stream, int64_t q_row0, int nq, uint64_t plant_stream,
                  uint64_t noise_stream, int64_t doc_id, int len, int d, double sigma, int dtype,
                  void *doc_rows, float *doc_scale);
int gen_codebook(uint64_t seed, uint64_t stream, int M, int K, int dsub, float *C);
int gen_codes(uint64_t seed, uint64_t stream, int64_t row0, int64_t n_tokens, int M, int K,
              uint8_t *codes);
int gen_encoded_codes(uint64_t seed, uint64_t stream, int64_t row0, int64_t n, int M, int K,
                      int dsub, const float *C, uint8_t *codes, int nthreads);
int gen_pq_encode(const double *x, int64_t n, int M, int K, int dsub, const float *C,
                  uint8_t *codes);
void gen_round_f32_to_bf16(const float *x, int64_t n, uint16_t *out);
void gen_round_f32_to_f16(const float *x, int64_t n, uint16_t *out);

/* oracle (oracle/maxsim_oracle.c) */
int oracle_maxsim_csr(const void *Q, int q_len, const void *D, const int64_t *offsets,
                      int64_t n_docs, int d, int dtype, double *out, int nthreads);
int oracle_maxsim_fixed(const void *Q, int q_len, const void *D, int64_t n_docs, int nd,
                        const int32_t *doc_lens, int d, int dtype, double *out, int nthreads);
int oracle_maxsim_argmax(const void *Q, int q_len, const void *D, const int64_t *offsets,
                         int64_t n_docs, int nd, int d, int dtype, double *out, double *tok_max,
                         int32_t *tok_arg, int nthreads);
int oracle_maxsim_backward(const void *Q, int q_len, const void *D, const int64_t *offsets,
                           int64_t n_docs, int nd, int d, int dtype, const int32_t *tok_arg,
                           const float *grad, double *dQ, double *dD);
int oracle_maxsim_i8(const int8_t *Q, const float *q_scale, int q_len, const int8_t *D,
                     const float *d_scale, const int64_t *offsets, int64_t n_docs, int nd, int d,
                     double *out, float *tok_max, int32_t *tok_arg, int nthreads);
int oracle_pq_tables(const void *Q, int q_len, int dtype, const float *C, int M, int K, int dsub,
                     double *T);
int oracle_maxsim_pq(const double *T, int q_len, int M, int K, const uint8_t *codes,
                     const int64_t *offsets, int64_t n_docs, int nd, double *out, int nthreads);

enum { BF16 = 0, FP16 = 1, FP32 = 2, I8 = 4 }; /* generator storage codes (oracle: 0..2) */

static int failures = 0;
static void check(int rc, const char *what) {
  if (rc != 0) {
    fprintf(stderr, "%s returned %d\n", what, rc);
    failures++;
  }
}
static void check_scores(const double *s, int64_t n, const int64_t *off, const char *what) {
  for (int64_t b = 0; b < n; b++) {
    const int empty = off && off[b + 1] == off[b];
    if (empty ? !(isinf(s[b]) && s[b] < 0) : !isfinite(s[b])) {
      fprintf(stderr, "%s: score %lld = %g\n", what, (long long)b, s[b]);
      failures++;
    }
  }
}

int main(void) {
  const int d = 64, q_len = 19, nthreads = 4;
  const int64_t n_docs = 23;
  const int elem[3] = {2, 2, 4};

  /* ragged CSR lengths with empty and one-token documents */
  int32_t lens[23];
  check(gen_lengths(5, 3, n_docs, 6.0, 0.8, 0, 20, lens), "gen_lengths");
  lens[0] = 0;
  lens[7] = 1;
  lens[22] = 0;
  int64_t off[24];
  off[0] = 0;
  for (int b = 0; b < n_docs; b++) off[b + 1] = off[b] + lens[b];
  const int64_t n_tok = off[n_docs];
  const int nd = 20; /* fixed layout: n_docs x nd, lens as the mask */

  for (int dt = BF16; dt <= FP32; dt++) {
    const size_t e = (size_t)elem[dt];
    void *Q = malloc((size_t)q_len * d * e);
    void *D = malloc((size_t)n_docs * nd * d * e); /* large enough for both layouts */
    check(gen_tokens(1, 0, 0, q_len, d, dt, Q, NULL, nthreads), "gen_tokens query");
    check(gen_tokens(1, 1, 0, n_docs * nd, d, dt, D, NULL, nthreads), "gen_tokens docs");
    check(gen_plant_doc(1, 0, 0, q_len, 2, 5, 3, nd, d, 0.05, dt, (char *)D + 3 * nd * d * e, NULL),
          "gen_plant_doc");
    check(gen_plant_doc(1, 0, 0, q_len, 2, 5, 7, 1, d, 0.05, dt, (char *)D + 7 * nd * d * e, NULL),
          "gen_plant_doc (one token)");
    double *out = malloc(sizeof(double) * n_docs);
    double *tmax = malloc(sizeof(double) * n_docs * q_len);
    int32_t *targ = malloc(sizeof(int32_t) * n_docs * q_len);
    check(oracle_maxsim_csr(Q, q_len, D, off, n_docs, d, dt, out, nthreads), "oracle csr");
    check_scores(out, n_docs, off, "oracle csr");
    check(oracle_maxsim_fixed(Q, q_len, D, n_docs, nd, lens, d, dt, out, nthreads), "oracle fixed");
    check_scores(out, n_docs, off, "oracle fixed (masked)");
    check(oracle_maxsim_fixed(Q, q_len, D, n_docs, nd, NULL, d, dt, out, nthreads),
          "oracle fixed (no mask)");
    check_scores(out, n_docs, NULL, "oracle fixed (no mask)");
    check(oracle_maxsim_argmax(Q, q_len, D, off, n_docs, 0, d, dt, out, tmax, targ, nthreads),
          "oracle argmax csr");
    float *g = malloc(sizeof(float) * n_docs);
    for (int b = 0; b < n_docs; b++) g[b] = (float)(b % 5) - 2.0f;
    double *dQ = malloc(sizeof(double) * q_len * d);
    double *dD = malloc(sizeof(double) * n_tok * d);
    check(oracle_maxsim_backward(Q, q_len, D, off, n_docs, 0, d, dt, targ, g, dQ, dD),
          "oracle backward csr");
    check(oracle_maxsim_backward(Q, q_len, D, off, n_docs, 0, d, dt, targ, g, NULL, dD),
          "oracle backward csr (dD only)");
    check(oracle_maxsim_argmax(Q, q_len, D, NULL, n_docs, nd, d, dt, out, tmax, targ, nthreads),
          "oracle argmax fixed");
    double *dDf = malloc(sizeof(double) * n_docs * nd * d);
    check(oracle_maxsim_backward(Q, q_len, D, NULL, n_docs, nd, d, dt, targ, g, dQ, NULL),
          "oracle backward fixed (dQ only)");
    check(oracle_maxsim_backward(Q, q_len, D, NULL, n_docs, nd, d, dt, targ, g, dQ, dDf),
          "oracle backward fixed");
    free(dDf);
    free(dQ);
    free(dD);
    free(g);
    free(tmax);
    free(targ);
    free(out);
    free(Q);
    free(D);
  }

  { /* INT8 with per-token scales, CSR and fixed, with and without per-token outputs */
    int8_t *Q = malloc((size_t)q_len * d);
    int8_t *D = malloc((size_t)n_docs * nd * d);
    float *qs = malloc(sizeof(float) * q_len), *ds = malloc(sizeof(float) * n_docs * nd);
    check(gen_tokens(4, 0, 0, q_len, d, I8, Q, qs, nthreads), "gen_tokens i8 query");
    check(gen_tokens(4, 1, 0, n_docs * nd, d, I8, D, ds, nthreads), "gen_tokens i8 docs");
    double *out = malloc(sizeof(double) * n_docs);
    float *tmax = malloc(sizeof(float) * n_docs * q_len);
    int32_t *targ = malloc(sizeof(int32_t) * n_docs * q_len);
    check(oracle_maxsim_i8(Q, qs, q_len, D, ds, off, n_docs, 0, d, out, tmax, targ, nthreads),
          "oracle i8 csr");
    check_scores(out, n_docs, off, "oracle i8 csr");
    check(oracle_maxsim_i8(Q, qs, q_len, D, ds, NULL, n_docs, nd, d, out, NULL, NULL, nthreads),
          "oracle i8 fixed");
    check_scores(out, n_docs, NULL, "oracle i8 fixed");
    free(Q);
    free(D);
    free(qs);
    free(ds);
    free(out);
    free(tmax);
    free(targ);
  }

  { /* PQ: codebook, encoding, uniform codes, tables, scoring */
    const int M = 8, K = 256, dsub = 8, dp = M * dsub;
    float *C = malloc(sizeof(float) * M * K * dsub);
    check(gen_codebook(5, 4, M, K, dsub, C), "gen_codebook");
    uint16_t *Q = malloc(sizeof(uint16_t) * q_len * dp);
    check(gen_tokens(5, 0, 0, q_len, dp, BF16, Q, NULL, nthreads), "gen_tokens pq query");
    uint8_t *codes = malloc((size_t)n_docs * nd * M);
    check(gen_codes(5, 6, 0, n_docs * nd, M, K, codes), "gen_codes");
    double *x = malloc(sizeof(double) * 3 * dp);
    for (int i = 0; i < 3 * dp; i++) x[i] = sin(0.37 * i);
    check(gen_pq_encode(x, 3, M, K, dsub, C, codes), "gen_pq_encode");
    check(gen_encoded_codes(5, 1, 0, n_docs * nd, M, K, dsub, C, codes, nthreads),
          "gen_encoded_codes");
    check(gen_encoded_codes(5, 1, 7, 0, M, K, dsub, C, codes, nthreads), "gen_encoded_codes n=0");
    double *T = malloc(sizeof(double) * q_len * M * K);
    check(oracle_pq_tables(Q, q_len, BF16, C, M, K, dsub, T), "oracle pq tables");
    double *out = malloc(sizeof(double) * n_docs);
    check(oracle_maxsim_pq(T, q_len, M, K, codes, off, n_docs, 0, out, nthreads), "oracle pq csr");
    check_scores(out, n_docs, off, "oracle pq csr");
    check(oracle_maxsim_pq(T, q_len, M, K, codes, NULL, n_docs, nd, out, nthreads),
          "oracle pq fixed");
    check_scores(out, n_docs, NULL, "oracle pq fixed");
    free(C);
    free(Q);
    free(codes);
    free(x);
    free(T);
    free(out);
  }

  { /* storage rounding helpers and distinct draws */
    float f[6] = {1.0f, -0.0f, 65504.0f, 1e-8f, 3.14159f, -2.5e-6f};
    uint16_t h[6];
    gen_round_f32_to_bf16(f, 6, h);
    gen_round_f32_to_f16(f, 6, h);
    int64_t pick[10];
    check(gen_distinct(1, 2, 9, 10, 10, pick), "gen_distinct");
  }

  if (failures) {
    fprintf(stderr, "sanitize driver: %d failures\n", failures);
    return 1;
  }
  printf("sanitize driver: ok\n");
  return 0;
}
