// Several short queries per pass on the one-wave-per-document kernel (bf16 / fp16 storage,
// rows of 128 or 256 bytes).
#include "dense_batch_kernel.hpp"
#include "dense_dispatch.hpp"

namespace maxsim {

namespace {

constexpr int DBATCH_G = 4;  // document tiles per group

template <int DT, int KSB, int NQB>
int launch_dense_batch(const DenseArgs &a, const DeviceInfo &di, hipStream_t st) {
  auto kern = dense_batch_kernel<DT, KSB, DBATCH_G, NQB>;
  const size_t lds = dense_batch_lds<KSB, NQB>();
  if (lds > di.max_lds) return MAXSIM_ERR_UNSUPPORTED;
  const int bpc = blocks_per_cu((const void *)kern, DBATCH_THREADS, lds);
  const int64_t max_wg = (int64_t)bpc * di.cus;
  const int64_t need = (a.n_docs + DBATCH_WAVES - 1) / DBATCH_WAVES;
  int64_t grid = need < max_wg ? need : max_wg;
  if (grid < 1) grid = 1;
  DenseArgs ka = a;
  // fixed documents: one contiguous range per wave once every wave gets at least 4
  ka.contiguous = !a.offsets && a.n_docs >= 4 * grid * DBATCH_WAVES;
  char what[64];
  std::snprintf(what, sizeof what, "dense_batch<DT=%d,KSB=%d,G=%d,NQB=%d>", DT, KSB, DBATCH_G, NQB);
  log_launch(what, (const void *)kern, grid, DBATCH_THREADS, lds, bpc);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(DBATCH_THREADS), lds, st, ka);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

template <int DT, int KSB>
int dense_batch_by_nqb(int nqb, const DenseArgs &a, const DeviceInfo &di, hipStream_t st) {
  switch ((nqb + 1) / 2) {  // an even number of blocks: at most one zero block
  case 1: return launch_dense_batch<DT, KSB, 2>(a, di, st);
  case 2: return launch_dense_batch<DT, KSB, 4>(a, di, st);
  case 3: return launch_dense_batch<DT, KSB, 6>(a, di, st);
  case 4: return launch_dense_batch<DT, KSB, 8>(a, di, st);
  case 5: return launch_dense_batch<DT, KSB, 10>(a, di, st);
  case 6: return launch_dense_batch<DT, KSB, 12>(a, di, st);
  case 7: return launch_dense_batch<DT, KSB, 14>(a, di, st);
  case 8: return launch_dense_batch<DT, KSB, 16>(a, di, st);
  }
  return MAXSIM_ERR_UNSUPPORTED;
}

template <int DT>
int dense_batch_by_ksb(int ksb, int nqb, const DenseArgs &a, const DeviceInfo &di, hipStream_t st) {
  switch (ksb) {
  case 2: return dense_batch_by_nqb<DT, 2>(nqb, a, di, st);
  case 4: return dense_batch_by_nqb<DT, 4>(nqb, a, di, st);
  }
  return MAXSIM_ERR_UNSUPPORTED;
}

}  // namespace

int dense_batch_blocks(int n_q, int q_len) { return n_q * ((q_len + 15) / 16); }

bool dense_batch_fits(int n_q, int q_len, int d, int dtype) {
  const int row = d * elem_bytes(dtype);
  return (dtype == MAXSIM_BF16 || dtype == MAXSIM_FP16) && (row == 128 || row == 256) &&
         dense_batch_blocks(n_q, q_len) <= DBATCH_MAX_BLOCKS;
}

int dense_batch_run(const DenseArgs &a, int d, int dtype, const DeviceInfo &di, hipStream_t st) {
  if (!dense_batch_fits(a.n_q, a.q_len, d, dtype)) return MAXSIM_ERR_UNSUPPORTED;
  const int ksb = d * elem_bytes(dtype) / 64, nqb = dense_batch_blocks(a.n_q, a.q_len);
  return dtype == MAXSIM_BF16 ? dense_batch_by_ksb<DT_BF16>(ksb, nqb, a, di, st)
                              : dense_batch_by_ksb<DT_FP16>(ksb, nqb, a, di, st);
}

}  // namespace maxsim
