// libmaxsim: the C-ABI entry points declared in include/maxsim.h.
//
// Each entry point checks its scalar and pointer arguments on the host,
// chooses a kernel variant from (dtype, d, q_len) and enqueues it on the
// caller's stream. Nothing here reads device memory or allocates.
#include <hip/hip_runtime.h>

#include "dense_dispatch.hpp"
#include "dense_kernel.hpp"
#include "host_common.hpp"
#include "tiled_dispatch.hpp"
#include "pq_kernel.hpp"

using namespace maxsim;

namespace {

// Pick and launch the dense kernel for validated arguments; with tok_max / tok_arg set the
// variant that also writes per-token maxima and argmax.
int dense_run(DenseArgs a, int d, int dtype, hipStream_t st) {
  const bool arg = a.tok_max != nullptr;
  DeviceInfo di;
  int rc = current_device(di);
  if (rc != MAXSIM_OK) return rc;
  const int eb = elem_bytes(dtype);
  const int chunks = d * eb / 64;          // 64-byte pieces per token row
  const int qb = (a.q_len + 15) / 16;      // 16-query blocks
  static const int force_lds = env_knob("MAXSIM_DENSE_QLDS", 0);
  // 5 to 16 query blocks of two-byte rows of 128 or 256 bytes (no per-token outputs): the
  // several-query kernel with one query, the query in LDS and each wave on one document.
  // MAXSIM_BATCH_DENSE=0 keeps them on the query-tiled kernel (for A/B measurements).
  static const int batch_ok = env_knob("MAXSIM_BATCH_DENSE", 1);
  if (qb > 4 && !arg && batch_ok && dense_batch_fits(1, a.q_len, d, dtype)) {
    a.n_q = 1;
    return dense_batch_run(a, d, dtype, di, st);
  }
  if (qb > 4) {
    // Long queries: query slices across the waves of a workgroup.
    TiledArgs t{a.Q, a.q_len, a.D, a.offsets, a.n_docs, a.nd, a.doc_lens, nullptr, nullptr,
                a.out, a.tok_max, a.tok_arg};
    return arg ? tiled_dense_argmax_run(t, d, dtype, di, st) : tiled_dense_run(t, d, dtype, di, st);
  }
  bool qlds = force_lds || chunks > 8 || chunks * qb > 16;
  int ksb = chunks;
  if (qlds) {
    ksb = 8;
    while (chunks % ksb) ksb--;
  }
  a.n_dblk = chunks / ksb;
  size_t lds = qlds ? (size_t)qb * 16 * ((size_t)d * eb + 16) : 0;
  if (lds > di.max_lds) return MAXSIM_ERR_UNSUPPORTED;
  switch (dtype) {
  case MAXSIM_BF16:
    return arg ? dense_argmax_dispatch_bf16(qlds, ksb, qb, a, lds, di, st)
               : dense_dispatch_bf16(qlds, ksb, qb, a, lds, di, st);
  case MAXSIM_FP16:
    return arg ? dense_argmax_dispatch_fp16(qlds, ksb, qb, a, lds, di, st)
               : dense_dispatch_fp16(qlds, ksb, qb, a, lds, di, st);
  case MAXSIM_FP32:
    return arg ? dense_argmax_dispatch_fp32(qlds, ksb, qb, a, lds, di, st)
               : dense_dispatch_fp32(qlds, ksb, qb, a, lds, di, st);
  }
  return MAXSIM_ERR_DTYPE;
}

}  // namespace

extern "C" {

int maxsim_score(const void *Q, int q_len, const void *D, const int64_t *doc_offsets,
                 int64_t n_docs, int d, int dtype, float *out, void *stream) {
  int rc = check_dense(Q, q_len, D, n_docs, d, dtype, out);
  if (rc != MAXSIM_OK) return rc;
  if (!doc_offsets) return MAXSIM_ERR_NULL;
  if (!aligned(doc_offsets, 8)) return MAXSIM_ERR_ALIGN;
  if (n_docs == 0) return MAXSIM_OK;
  DenseArgs a{(const char *)Q, q_len, (const char *)D, doc_offsets, n_docs, 0, nullptr, 1, out};
  return dense_run(a, d, dtype, (hipStream_t)stream);
}

int maxsim_score_fixed(const void *Q, int q_len, const void *D, int64_t n_docs, int nd,
                       const int32_t *doc_lens, int d, int dtype, float *out, void *stream) {
  int rc = check_dense(Q, q_len, D, n_docs, d, dtype, out);
  if (rc != MAXSIM_OK) return rc;
  if (nd < 1) return MAXSIM_ERR_SHAPE;
  if (doc_lens && !aligned(doc_lens, 4)) return MAXSIM_ERR_ALIGN;
  if (n_docs == 0) return MAXSIM_OK;
  DenseArgs a{(const char *)Q, q_len, (const char *)D, nullptr, n_docs, nd, doc_lens, 1, out};
  return dense_run(a, d, dtype, (hipStream_t)stream);
}

int maxsim_score_argmax(const void *Q, int q_len, const void *D, const int64_t *doc_offsets,
                        int64_t n_docs, int nd, int d, int dtype, float *out, float *tok_max,
                        int32_t *tok_arg, void *stream) {
  int rc = check_dense(Q, q_len, D, n_docs, d, dtype, out);
  if (rc != MAXSIM_OK) return rc;
  if (!doc_offsets && nd < 1) return MAXSIM_ERR_SHAPE;
  if (!tok_max || !tok_arg) return MAXSIM_ERR_NULL;
  if ((doc_offsets && !aligned(doc_offsets, 8)) || !aligned(tok_max, 4) || !aligned(tok_arg, 4))
    return MAXSIM_ERR_ALIGN;
  if (n_docs == 0) return MAXSIM_OK;
  DenseArgs a{(const char *)Q, q_len,   (const char *)D, doc_offsets, n_docs,
              doc_offsets ? 0 : nd,   nullptr, 1,          out,         tok_max, tok_arg};
  return dense_run(a, d, dtype, (hipStream_t)stream);
}

int maxsim_score_batch(const void *Q, int n_q, int q_len, const void *D,
                       const int64_t *doc_offsets, int64_t n_docs, int nd, int d, int dtype,
                       float *out, void *stream) {
  int rc = check_dense(Q, q_len, D, n_docs, d, dtype, out);
  if (rc != MAXSIM_OK) return rc;
  if (n_q < 1 || (!doc_offsets && nd < 1)) return MAXSIM_ERR_SHAPE;
  if (doc_offsets && !aligned(doc_offsets, 8)) return MAXSIM_ERR_ALIGN;
  const int ksb = d * elem_bytes(dtype) / 64;
  if (d * elem_bytes(dtype) % 64 != 0 || (ksb != 1 && ksb != 2 && ksb != 4 && ksb != 8))
    return MAXSIM_ERR_UNSUPPORTED;
  const int q_pad = (q_len + 15) & ~15;
  const int group = tiled_max_q(ksb) / q_pad;  // queries per pass over the documents
  if (group < 1) return MAXSIM_ERR_UNSUPPORTED;
  if (n_docs == 0) return MAXSIM_OK;
  if (n_q == 1) {
    // the single-query kernels, so that a batch of one equals maxsim_score bit for bit
    DenseArgs a{(const char *)Q, q_len, (const char *)D, doc_offsets, n_docs,
                doc_offsets ? 0 : nd, nullptr, 1, out};
    return dense_run(a, d, dtype, (hipStream_t)stream);
  }
  DeviceInfo di;
  rc = current_device(di);
  if (rc != MAXSIM_OK) return rc;
  // Up to 16 blocks of query tokens (two-byte rows of 128 or 256 bytes): the
  // one-wave-per-document kernel with the queries in LDS. MAXSIM_BATCH_DENSE=0 forces the
  // query-tiled kernel (for A/B measurements).
  static const int dense_ok = env_knob("MAXSIM_BATCH_DENSE", 1);
  if (dense_ok && dense_batch_fits(n_q, q_len, d, dtype)) {
    DenseArgs a{(const char *)Q, q_len, (const char *)D, doc_offsets, n_docs,
                doc_offsets ? 0 : nd, nullptr, 1, out};
    a.n_q = n_q;
    return dense_batch_run(a, d, dtype, di, (hipStream_t)stream);
  }
  const int64_t q_bytes = (int64_t)q_len * d * elem_bytes(dtype);
  for (int q0 = 0; q0 < n_q; q0 += group) {
    TiledArgs a{(const char *)Q + q0 * q_bytes, q_len, (const char *)D, doc_offsets, n_docs,
                doc_offsets ? 0 : nd, nullptr, nullptr, nullptr, out + (int64_t)q0 * n_docs,
                nullptr, nullptr, n_q - q0 < group ? n_q - q0 : group};
    rc = tiled_batch_run(a, d, dtype, di, (hipStream_t)stream);
    if (rc != MAXSIM_OK) return rc;
  }
  return MAXSIM_OK;
}

int maxsim_score_i8(const int8_t *Q, const float *q_scale, int q_len, const int8_t *D,
                    const float *d_scale, const int64_t *doc_offsets, int64_t n_docs, int nd,
                    int d, float *out, float *tok_max, int32_t *tok_arg, void *stream) {
  if (n_docs < 0 || q_len < 1 || q_len > MAXSIM_MAX_Q_LEN) return MAXSIM_ERR_SHAPE;
  if (d < 64 || d > MAXSIM_MAX_D || d % 64 != 0) return MAXSIM_ERR_SHAPE;
  if (!doc_offsets && nd < 1) return MAXSIM_ERR_SHAPE;
  if (!Q || !q_scale || !D || !d_scale || !out) return MAXSIM_ERR_NULL;
  if ((tok_max == nullptr) != (tok_arg == nullptr)) return MAXSIM_ERR_NULL;
  if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(q_scale, 4) || !aligned(d_scale, 4) ||
      !aligned(out, 4) || (doc_offsets && !aligned(doc_offsets, 8)) ||
      (tok_max && (!aligned(tok_max, 4) || !aligned(tok_arg, 4))))
    return MAXSIM_ERR_ALIGN;
  if (n_docs == 0) return MAXSIM_OK;
  DeviceInfo di;
  int rc = current_device(di);
  if (rc != MAXSIM_OK) return rc;
  if (q_len <= 64 && (d == 64 || d == 128 || d == 256)) {
    // One wave per document with the query in registers, as for 16-bit storage: the
    // document stream, not the matrix core, bounds these shapes.
    DenseArgs a{(const char *)Q, q_len, (const char *)D, doc_offsets, n_docs,
                doc_offsets ? 0 : nd, nullptr, 1, out, tok_max, tok_arg};
    a.q_scale = q_scale;
    a.d_scale = d_scale;
    return dense_i8_run(d / 64, (q_len + 15) / 16, a, di, (hipStream_t)stream);
  }
  TiledArgs a{(const char *)Q, q_len, (const char *)D, doc_offsets, n_docs, nd, nullptr, q_scale,
              d_scale, out, tok_max, tok_arg};
  return tiled_i8_run(a, d, di, (hipStream_t)stream);
}

int maxsim_pq_tables(const void *Q, int q_len, int dtype, const float *C, int M, int K, int dsub,
                     float *T, void *stream) {
  if (elem_bytes(dtype) == 0) return MAXSIM_ERR_DTYPE;
  if (q_len < 1 || q_len > MAXSIM_MAX_Q_LEN || M < 1 || dsub < 1 || dsub > 32)
    return MAXSIM_ERR_SHAPE;
  const int d = M * dsub;
  if (d < MAXSIM_MIN_D || d > MAXSIM_MAX_D || d % 32 != 0) return MAXSIM_ERR_SHAPE;
  if (K != 256) return MAXSIM_ERR_UNSUPPORTED;
  if (!Q || !C || !T) return MAXSIM_ERR_NULL;
  if (!aligned(Q, 16) || !aligned(C, 16) || !aligned(T, 16)) return MAXSIM_ERR_ALIGN;
  DeviceInfo di;
  int rc = current_device(di);
  if (rc != MAXSIM_OK) return rc;
  PqTableArgs a{(const char *)Q, q_len, dtype, C, M, K, dsub, T};
  return pq_tables_run(a, di, (hipStream_t)stream);
}

int maxsim_score_pq(const float *T, int q_len, int M, int K, const uint8_t *codes,
                    const int64_t *doc_offsets, int64_t n_docs, int nd, float *out, void *stream) {
  if (n_docs < 0 || q_len < 1 || q_len > MAXSIM_MAX_Q_LEN || M < 1) return MAXSIM_ERR_SHAPE;
  if (!doc_offsets && nd < 1) return MAXSIM_ERR_SHAPE;
  if (K != 256 || M != 16 || q_len > PQ_MAX_Q) return MAXSIM_ERR_UNSUPPORTED;
  if (!T || !codes || !out) return MAXSIM_ERR_NULL;
  if (!aligned(T, 16) || !aligned(codes, 16) || !aligned(out, 4) ||
      (doc_offsets && !aligned(doc_offsets, 8)))
    return MAXSIM_ERR_ALIGN;
  if (n_docs == 0) return MAXSIM_OK;
  DeviceInfo di;
  int rc = current_device(di);
  if (rc != MAXSIM_OK) return rc;
  PqScoreArgs a{T, q_len, codes, doc_offsets, n_docs, nd, out};
  return pq_score_run(a, di, (hipStream_t)stream);
}

const char *maxsim_status_string(int status) {
  switch (status) {
  case MAXSIM_OK: return "ok";
  case MAXSIM_ERR_NULL: return "a required pointer is NULL";
  case MAXSIM_ERR_SHAPE: return "a size argument is out of range";
  case MAXSIM_ERR_DTYPE: return "unknown dtype";
  case MAXSIM_ERR_ALIGN: return "a pointer is not aligned as required";
  case MAXSIM_ERR_UNSUPPORTED: return "no kernel for this combination of sizes";
  case MAXSIM_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
  case MAXSIM_ERR_DEVICE: return "no gfx950 device is current";
  case MAXSIM_ERR_SCRATCH: return "the call needs more than the library's static scratch memory";
  }
  return "unknown status";
}

int maxsim_version(void) { return 100; }

}  // extern "C"
