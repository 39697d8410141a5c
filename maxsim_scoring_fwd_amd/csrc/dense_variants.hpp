// Dense kernel variants and their launch (included once per storage type).
#pragma once

#include "dense_dispatch.hpp"

namespace maxsim {
namespace {

constexpr int DENSE_WAVES_PER_WG = DENSE_THREADS / WAVE;

template <int DT, int KSB, int QB, int P, bool QLDS>
int launch_dense(const DenseArgs &a, size_t lds, const DeviceInfo &di, hipStream_t st) {
  auto kern = dense_maxsim_kernel<DT, KSB, QB, P, QLDS>;
  const int bpc = blocks_per_cu((const void *)kern, DENSE_THREADS, lds);
  const int64_t max_wg = (int64_t)bpc * di.cus;
  const int64_t need = (a.n_docs + DENSE_WAVES_PER_WG - 1) / DENSE_WAVES_PER_WG;
  int64_t grid = need < max_wg ? need : max_wg;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(DENSE_THREADS), lds, st, a);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

// Tiles in flight per wave: about 32 KiB of loads per wave for small chunks counts.
template <int KSB> constexpr int default_depth() { return KSB <= 4 ? 8 : 4; }

template <int DT, int KSB, int QB, bool QLDS>
int dense_with_depth(const DenseArgs &a, size_t lds, const DeviceInfo &di, hipStream_t st) {
  if constexpr (DT == DT_BF16 && KSB == 4 && QB == 2 && !QLDS) {
    // The ColBERT shape (d = 128, 32 query tokens): depth selectable for measurements.
    static const int depth = env_knob("MAXSIM_DENSE_DEPTH", 0);
    if (depth == 2) return launch_dense<DT, KSB, QB, 2, QLDS>(a, lds, di, st);
    if (depth == 4) return launch_dense<DT, KSB, QB, 4, QLDS>(a, lds, di, st);
    if (depth == 12) return launch_dense<DT, KSB, QB, 12, QLDS>(a, lds, di, st);
  }
  return launch_dense<DT, KSB, QB, default_depth<KSB>(), QLDS>(a, lds, di, st);
}

template <int DT, int KSB, bool QLDS>
int dense_by_qb(int qb, const DenseArgs &a, size_t lds, const DeviceInfo &di, hipStream_t st) {
  // Register-resident queries only while Q needs at most 64 VGPRs.
  switch (qb) {
  case 1: return dense_with_depth<DT, KSB, 1, QLDS>(a, lds, di, st);
  case 2: return dense_with_depth<DT, KSB, 2, QLDS>(a, lds, di, st);
  case 3:
    if constexpr (QLDS || KSB * 3 <= 16) return dense_with_depth<DT, KSB, 3, QLDS>(a, lds, di, st);
    break;
  case 4:
    if constexpr (QLDS || KSB * 4 <= 16) return dense_with_depth<DT, KSB, 4, QLDS>(a, lds, di, st);
    break;
  }
  return MAXSIM_ERR_UNSUPPORTED;
}

template <int DT, bool QLDS>
int dense_by_ksb(int ksb, int qb, const DenseArgs &a, size_t lds, const DeviceInfo &di,
                 hipStream_t st) {
  switch (ksb) {
  case 1: return dense_by_qb<DT, 1, QLDS>(qb, a, lds, di, st);
  case 2: return dense_by_qb<DT, 2, QLDS>(qb, a, lds, di, st);
  case 3: return dense_by_qb<DT, 3, QLDS>(qb, a, lds, di, st);
  case 4: return dense_by_qb<DT, 4, QLDS>(qb, a, lds, di, st);
  case 5: return dense_by_qb<DT, 5, QLDS>(qb, a, lds, di, st);
  case 6: return dense_by_qb<DT, 6, QLDS>(qb, a, lds, di, st);
  case 7: return dense_by_qb<DT, 7, QLDS>(qb, a, lds, di, st);
  case 8: return dense_by_qb<DT, 8, QLDS>(qb, a, lds, di, st);
  }
  return MAXSIM_ERR_UNSUPPORTED;
}

template <int DT>
int dense_by_mode(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds, const DeviceInfo &di,
                  hipStream_t st) {
  return qlds ? dense_by_ksb<DT, true>(ksb, qb, a, lds, di, st)
              : dense_by_ksb<DT, false>(ksb, qb, a, lds, di, st);
}

}  // namespace
}  // namespace maxsim
