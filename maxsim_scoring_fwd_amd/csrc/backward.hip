// libmaxsim backward entry points (include/maxsim.h): gradients of sum_b g_b * score_b
// from the forward argmax.
#include <hip/hip_runtime.h>

#include "backward_kernel.hpp"
#include "host_common.hpp"

using namespace maxsim;

namespace {

// Segment length of the inverse grid: a fixed-layout document in one segment where it
// fits, CSR documents (unknown lengths on the host) in segments of 256 tokens.
inline int dd_seg_cap(const BwdArgs &a) {
  if (a.offsets) return 256;
  const int r = (a.nd + WAVE - 1) / WAVE * WAVE;
  return r < BWD_SEG ? r : BWD_SEG;
}

template <int DT, int OT, bool QLDS>
int launch_dd_lds(const BwdArgs &a, int seg_cap, int q_lds, const DeviceInfo &di,
                  hipStream_t st) {
  // Workgroups per CU: fixed-length documents with the query in LDS write fastest from two
  // workgroups per CU (measured 5.45 against 5.06 TB/s at as many as fit: fewer streams of
  // stores); CSR documents and long queries need every resident wave to hide the latency
  // of their per-document phases. Non-temporal stores: the gradient rows are not re-read
  // (ordinary stores measured 0.1 ms slower per training step at the ColBERT shape). Knobs
  // override both for measurements.
  static const int nt = env_knob("MAXSIM_BWD_NT", 1);
  static const int wgs = env_knob("MAXSIM_BWD_WGS", -1);
  // CSR ranges balance 64 tokens per document plus one per token: the per-document phases
  // (counting, scan, placement) cost about as much as writing 64 gradient rows (measured
  // weights 0 / 16 / 32 / 64 / 128: 0.466 / 0.459-0.460 / 0.453-0.457 / 0.453-0.457 /
  // 0.453-0.454 ms at the lognormal corpus). MAXSIM_BWD_DOC_WEIGHT overrides it.
  static const int doc_weight = env_knob("MAXSIM_BWD_DOC_WEIGHT", 64);
  // Chosen-token sets for queries of at most 64 tokens (query in LDS): CSR dD measured
  // 0.429 against 0.454 ms at the lognormal corpus; fixed 128-token documents, capped at two
  // workgroups per CU, measured 0.640 against 0.591 ms, so they keep the counting path.
  // Prefetching the next document measured the same as loading it after the stores.
  // MAXSIM_BWD_SETS overrides (0 off, 1 sets, 3 sets without prefetch).
  static const int sets_knob = env_knob("MAXSIM_BWD_SETS", -1);
  const int short_sets = sets_knob >= 0 ? sets_knob : (a.offsets ? 1 : 0);
  auto kern = nt ? bwd_dd_kernel<DT, OT, QLDS, true> : bwd_dd_kernel<DT, OT, QLDS, false>;
  const size_t lds = (size_t)q_lds + (size_t)BWD_WAVES * bwd_dd_wave_ints(seg_cap, a.q_len) * 4;
  if (lds > di.max_lds) return MAXSIM_ERR_UNSUPPORTED;
  int bpc = blocks_per_cu((const void *)kern, BWD_THREADS, lds);
  const int cap = wgs >= 0 ? wgs : (QLDS && !a.offsets ? 2 : 0);
  if (cap > 0 && cap < bpc) bpc = cap;
  const int64_t max_wg = (int64_t)bpc * di.cus;
  const int64_t need = (a.n_docs + BWD_WAVES - 1) / BWD_WAVES;
  int64_t grid = need < max_wg ? need : max_wg;
  if (grid < 1) grid = 1;
  BwdArgs ka = a;
  ka.doc_weight = doc_weight;
  ka.short_sets = short_sets;
  log_launch(QLDS ? "bwd_dd<QLDS>" : "bwd_dd", (const void *)kern, grid, BWD_THREADS, lds, bpc);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(BWD_THREADS), lds, st, ka, seg_cap, q_lds);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

template <int DT, int OT>
int launch_dd(const BwdArgs &a, const DeviceInfo &di, hipStream_t st) {
  const int seg_cap = dd_seg_cap(a);
  const int q_bytes = a.q_len * a.d * Elem<DT>::bytes;  // a multiple of 64 (d % 32 == 0)
  if (q_bytes <= BWD_Q_LDS_MAX) return launch_dd_lds<DT, OT, true>(a, seg_cap, q_bytes, di, st);
  return launch_dd_lds<DT, OT, false>(a, seg_cap, 0, di, st);
}

template <int DT, int OT>
int launch_dq(const BwdArgs &a, hipStream_t st) {
  const unsigned blocks = (unsigned)((a.q_len * a.d + DQ_ELEMS_PER_WG - 1) / DQ_ELEMS_PER_WG);
  // Documents in flight per step of a thread; MAXSIM_BWD_DQ_DOCS (1, 2, 3, 4 or 8) overrides.
  static const int docs = env_knob("MAXSIM_BWD_DQ_DOCS", DQ_DOCS);
  auto kern = docs == 8   ? bwd_dq_partial_kernel<DT, 8>
              : docs == 3 ? bwd_dq_partial_kernel<DT, 3>
              : docs == 2 ? bwd_dq_partial_kernel<DT, 2>
              : docs == 1 ? bwd_dq_partial_kernel<DT, 1>
                          : bwd_dq_partial_kernel<DT, 4>;
  hipLaunchKernelGGL(kern, dim3(blocks, (unsigned)a.n_ranges), dim3(BWD_THREADS), 0, st, a);
  if (hipGetLastError() != hipSuccess) return MAXSIM_ERR_LAUNCH;
  const int n_elem = a.q_len * a.d;
  const unsigned rblocks = (unsigned)((n_elem + RED_ELEMS - 1) / RED_ELEMS);
  hipLaunchKernelGGL(bwd_dq_reduce_kernel<OT>, dim3(rblocks), dim3(BWD_THREADS), 0, st,
                     (const float *)a.partial, a.n_ranges, n_elem, a.dQ);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

// dQ = 0 in the gradient type: the range sum over no ranges stores 0 in every element.
int zero_dq(void *dQ, int n_elem, int grad_dtype, hipStream_t st) {
  const unsigned rblocks = (unsigned)((n_elem + RED_ELEMS - 1) / RED_ELEMS);
  auto kern = grad_dtype == MAXSIM_FP32   ? bwd_dq_reduce_kernel<DT_FP32>
              : grad_dtype == MAXSIM_BF16 ? bwd_dq_reduce_kernel<DT_BF16>
                                          : bwd_dq_reduce_kernel<DT_FP16>;
  hipLaunchKernelGGL(kern, dim3(rblocks), dim3(BWD_THREADS), 0, st, (const float *)nullptr, 0,
                     n_elem, (char *)dQ);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

int run_dd(const BwdArgs &a, int dtype, int grad_dtype, const DeviceInfo &di, hipStream_t st) {
  const bool f32 = grad_dtype == MAXSIM_FP32;
  switch (dtype) {
  case MAXSIM_BF16:
    return f32 ? launch_dd<DT_BF16, DT_FP32>(a, di, st) : launch_dd<DT_BF16, DT_BF16>(a, di, st);
  case MAXSIM_FP16:
    return f32 ? launch_dd<DT_FP16, DT_FP32>(a, di, st) : launch_dd<DT_FP16, DT_FP16>(a, di, st);
  case MAXSIM_FP32: return launch_dd<DT_FP32, DT_FP32>(a, di, st);
  }
  return MAXSIM_ERR_DTYPE;
}

int run_dq(const BwdArgs &a, int dtype, int grad_dtype, hipStream_t st) {
  const bool f32 = grad_dtype == MAXSIM_FP32;
  switch (dtype) {
  case MAXSIM_BF16:
    return f32 ? launch_dq<DT_BF16, DT_FP32>(a, st) : launch_dq<DT_BF16, DT_BF16>(a, st);
  case MAXSIM_FP16:
    return f32 ? launch_dq<DT_FP16, DT_FP32>(a, st) : launch_dq<DT_FP16, DT_FP16>(a, st);
  case MAXSIM_FP32: return launch_dq<DT_FP32, DT_FP32>(a, st);
  }
  return MAXSIM_ERR_DTYPE;
}

}  // namespace

extern "C" {

size_t maxsim_backward_workspace_size(int q_len, int d, int64_t n_docs) {
  if (q_len < 1 || q_len > MAXSIM_MAX_Q_LEN || d < MAXSIM_MIN_D || d > MAXSIM_MAX_D ||
      d % 32 != 0 || n_docs < 1)
    return 0;
  return (size_t)bwd_dq_ranges(q_len, d, n_docs) * (size_t)q_len * (size_t)d * sizeof(float);
}

int maxsim_backward(const void *Q, int q_len, const void *D, const int64_t *doc_offsets,
                    int64_t n_docs, int nd, int d, int dtype, const int32_t *tok_arg,
                    const float *grad_out, void *dQ, void *dD, int grad_dtype, void *workspace,
                    size_t workspace_bytes, void *stream) {
  if (elem_bytes(dtype) == 0) return MAXSIM_ERR_DTYPE;
  if (grad_dtype != MAXSIM_FP32 && grad_dtype != dtype) return MAXSIM_ERR_DTYPE;
  if (n_docs < 0 || q_len < 1 || q_len > MAXSIM_MAX_Q_LEN) return MAXSIM_ERR_SHAPE;
  if (d < MAXSIM_MIN_D || d > MAXSIM_MAX_D || d % 32 != 0) return MAXSIM_ERR_SHAPE;
  if (!doc_offsets && nd < 1) return MAXSIM_ERR_SHAPE;
  // with no documents, D, tok_arg and grad_out are empty and may be NULL
  if (!Q || (n_docs > 0 && (!D || !tok_arg || !grad_out))) return MAXSIM_ERR_NULL;
  if (dQ && !workspace) return MAXSIM_ERR_NULL;
  if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(tok_arg, 4) || !aligned(grad_out, 4) ||
      (doc_offsets && !aligned(doc_offsets, 8)) || (dQ && !aligned(dQ, 16)) ||
      (dD && !aligned(dD, 16)) || (workspace && !aligned(workspace, 16)))
    return MAXSIM_ERR_ALIGN;
  if (!dQ && !dD) return MAXSIM_OK;
  if (dQ && workspace_bytes < maxsim_backward_workspace_size(q_len, d, n_docs))
    return MAXSIM_ERR_SHAPE;
  if (n_docs == 0 && !dQ) return MAXSIM_OK;  // no rows of dD to write
  DeviceInfo di;
  int rc = current_device(di);
  if (rc != MAXSIM_OK) return rc;
  // No documents: the loss is an empty sum and dQ is zero (dD has no rows).
  if (n_docs == 0) return zero_dq(dQ, q_len * d, grad_dtype, (hipStream_t)stream);
  BwdArgs a{(const char *)Q, q_len, (const char *)D, doc_offsets, n_docs, doc_offsets ? 0 : nd, d,
            tok_arg, grad_out, (char *)dQ, (char *)dD, (float *)workspace,
            bwd_dq_ranges(q_len, d, n_docs)};
  hipStream_t st = (hipStream_t)stream;
  if (dD) {
    rc = run_dd(a, dtype, grad_dtype, di, st);
    if (rc != MAXSIM_OK) return rc;
  }
  if (dQ) return run_dq(a, dtype, grad_dtype, st);
  return MAXSIM_OK;
}

}  // extern "C"
