// Dense kernel variants and their launch (included once per storage type).
#pragma once

#include "dense_dispatch.hpp"

namespace maxsim {
namespace {

template <int DT, int KSB, int QB, int P, bool QLDS, int LM, bool ARG>
int launch_dense(const DenseArgs &a, size_t q_lds, const DeviceInfo &di, hipStream_t st) {
  auto kern = dense_maxsim_kernel<DT, KSB, QB, P, QLDS, LM, ARG>;
  const size_t lds = q_lds + (LM == LOAD_STAGED ? DENSE_WAVES * stage_tile_bytes<KSB>() : 0);
  if (lds > di.max_lds) return MAXSIM_ERR_UNSUPPORTED;
  int bpc = blocks_per_cu((const void *)kern, DENSE_THREADS, lds);
  // Fewer concurrent document streams read faster once each wave has a long range of
  // documents: bf16 / fp16 fixed documents of at least 32 KiB stream best from one
  // workgroup per CU (one wave per SIMD; 100K ColBERT documents 0.489 -> 0.478 ms, 500K
  // +2.7%, any query of 16-64 tokens alike; with per-token outputs 0.556 -> 0.533 ms),
  // 16 KiB documents from two (+1.2-1.7%), provided every wave still gets at least 32
  // documents (10K documents are fastest uncapped). fp32, 512-byte rows and the query in LDS
  // keep the full occupancy (measured no better or slower); INT8 below. MAXSIM_DENSE_WG_PER_CU
  // =n forces a cap of n, 0 none.
  static const int wg_env = env_knob("MAXSIM_DENSE_WG_PER_CU", -1);
  int wg_cap = 0;
  if constexpr ((DT == DT_BF16 || DT == DT_FP16) && !QLDS && (KSB == 2 || KSB == 4)) {
    const int64_t doc_bytes = (int64_t)a.nd * KSB * 64;
    const int64_t per_wave = 32 * (int64_t)di.cus * DENSE_WAVES;  // documents at one WG per CU
    if (!a.offsets && doc_bytes >= 32768 && a.n_docs >= per_wave)
      wg_cap = 1;
    else if (!a.offsets && doc_bytes >= 16384 && a.n_docs >= 2 * per_wave)
      wg_cap = 2;
  }
  if constexpr (DT == DT_I8 && KSB == 2 && !QLDS) {
    // INT8 rows of 128 bytes (depth 4, up to 5 workgroups per CU): three per CU, 80.5-80.8
    // -> 82.0-82.2% of HBM peak at 100K documents (one per CU 61%, two unsteady)
    if (!a.offsets && a.n_docs >= 3 * 32 * (int64_t)di.cus * DENSE_WAVES) wg_cap = 3;
  }
  if (wg_env >= 0) wg_cap = wg_env;
  if (wg_cap > 0 && wg_cap < bpc) bpc = wg_cap;
  const int64_t max_wg = (int64_t)bpc * di.cus;
  const int64_t need = (a.n_docs + DENSE_WAVES - 1) / DENSE_WAVES;
  int64_t grid = need < max_wg ? need : max_wg;
  if (grid < 1) grid = 1;
  // Fixed-length documents: with at least 4 documents per wave, each wave streams one
  // contiguous range of documents (measured +1-1.5 points of HBM peak for 16 KiB documents);
  // with fewer, the grid stride is faster (B = 10K: 73-74% against 71%). The forward with
  // argmax keeps the stride (2% faster at 100K ColBERT documents: neighbouring waves write
  // neighbouring rows of per-token outputs). MAXSIM_DENSE_CONTIG=0 / 1 forces either.
  static const int contig = env_knob("MAXSIM_DENSE_CONTIG", -1);
  DenseArgs ka = a;
  ka.contiguous = contig >= 0 ? contig : !ARG && a.n_docs >= 4 * grid * DENSE_WAVES;
  if (a.offsets) ka.contiguous = 0;
  char what[96];
  std::snprintf(what, sizeof what, "dense<DT=%d,KSB=%d,QB=%d,P=%d,QLDS=%d,LM=%d,ARG=%d>", DT, KSB,
                QB, P, (int)QLDS, LM, (int)ARG);
  log_launch(what, (const void *)kern, grid, DENSE_THREADS, lds, bpc);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(DENSE_THREADS), lds, st, ka);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

// Staged loads need a power-of-two number of 16-byte pieces per row.
template <int KSB> constexpr bool stageable() { return (KSB & (KSB - 1)) == 0; }

// Tiles in flight per wave. On the ColBERT shape depths 4 to 10 are within 1% of each other
// and 4 needs the fewest registers. Short rows, measured at 100K documents of 128 tokens
// against the former depth 8 (whose per-slot state spilled scalar registers): bf16 rows of
// 128 bytes (d = 64) 83.0 -> 85.1% of HBM peak at depth 4, of 64 bytes (d = 32) 0.143 ->
// 0.139 ms; INT8 rows of 128 bytes +0.7% at depth 4, of 64 bytes 0.156 -> 0.151-0.154 ms at
// depth 6 (depth 4 slower there). fp32 short rows keep 8 (not measured).
template <int DT, int KSB> constexpr int default_depth() {
  if constexpr (DT == DT_I8) return KSB == 1 ? 6 : 4;
  else if constexpr (DT == DT_FP32) return KSB <= 2 ? 8 : 4;
  else return 4;
}

template <int DT, int KSB, int QB, bool QLDS, bool ARG>
int dense_with_depth(const DenseArgs &a, size_t lds, const DeviceInfo &di, hipStream_t st) {
  constexpr int LM = stageable<KSB>() ? LOAD_STAGED : LOAD_DIRECT;
  if constexpr (DT == DT_BF16 && KSB == 4 && QB == 2 && !ARG) {
    // The ColBERT shape (d = 128, 32 query tokens): load mode, ring depth and query
    // placement selectable for measurements.
    static const int depth = env_knob("MAXSIM_DENSE_DEPTH", 0);
    static const int mode = env_knob("MAXSIM_DENSE_LOAD", LM);
    if constexpr (!QLDS) {
      if (mode == LOAD_DIRECT) {
        if (depth == 12) return launch_dense<DT, KSB, QB, 12, QLDS, LOAD_DIRECT, ARG>(a, lds, di, st);
        return launch_dense<DT, KSB, QB, 8, QLDS, LOAD_DIRECT, ARG>(a, lds, di, st);
      }
      if (mode == LOAD_DIRECT_NT)
        return launch_dense<DT, KSB, QB, 8, QLDS, LOAD_DIRECT_NT, ARG>(a, lds, di, st);
    }
    // CSR corpora: token-balanced ranges end on document boundaries, so a wave whose range
    // ends inside a long document finishes last, alone; a deeper ring shortens that tail
    // (measured depth 4 / 6 / 10 / 12: 80.5-80.7 / 80.7-81.0 / 81.2-81.4 / 81.8-81.9% of
    // HBM peak on the lognormal corpus). At depth 12 the kernel takes 253 VGPRs and 8 AGPRs,
    // so it runs one wave per SIMD (one workgroup per CU): twelve tiles in flight per SIMD,
    // as at depth 4 with three waves per SIMD, but from a single wave.
    if (a.offsets && depth == 0)
      return launch_dense<DT, KSB, QB, 12, QLDS, LOAD_STAGED, ARG>(a, lds, di, st);
    if (depth == 4) return launch_dense<DT, KSB, QB, 4, QLDS, LOAD_STAGED, ARG>(a, lds, di, st);
    if (depth == 6) return launch_dense<DT, KSB, QB, 6, QLDS, LOAD_STAGED, ARG>(a, lds, di, st);
    if (depth == 10) return launch_dense<DT, KSB, QB, 10, QLDS, LOAD_STAGED, ARG>(a, lds, di, st);
    if (depth == 12) return launch_dense<DT, KSB, QB, 12, QLDS, LOAD_STAGED, ARG>(a, lds, di, st);
  }
  if constexpr ((DT == DT_BF16 || DT == DT_I8) && KSB <= 2 && QB == 2 && !ARG && !QLDS) {
    // rows of 64 or 128 bytes with 32 query tokens: ring depth selectable for measurements
    static const int depth = env_knob("MAXSIM_DENSE_DEPTH", 0);
    if (depth == 4) return launch_dense<DT, KSB, QB, 4, QLDS, LM, ARG>(a, lds, di, st);
    if (depth == 6) return launch_dense<DT, KSB, QB, 6, QLDS, LM, ARG>(a, lds, di, st);
    if (depth == 8) return launch_dense<DT, KSB, QB, 8, QLDS, LM, ARG>(a, lds, di, st);
    if (depth == 12) return launch_dense<DT, KSB, QB, 12, QLDS, LM, ARG>(a, lds, di, st);
  }
  if constexpr (LM == LOAD_STAGED) {
    // Where Q already fills LDS, the transpose buffers may not fit: load directly.
    if (lds + DENSE_WAVES * stage_tile_bytes<KSB>() > di.max_lds)
      return launch_dense<DT, KSB, QB, default_depth<DT, KSB>(), QLDS, LOAD_DIRECT, ARG>(a, lds, di, st);
  }
  return launch_dense<DT, KSB, QB, default_depth<DT, KSB>(), QLDS, LM, ARG>(a, lds, di, st);
}

template <int DT, int KSB, bool QLDS, bool ARG>
int dense_by_qb(int qb, const DenseArgs &a, size_t lds, const DeviceInfo &di, hipStream_t st) {
  // Register-resident queries only while Q needs at most 64 VGPRs.
  switch (qb) {
  case 1: return dense_with_depth<DT, KSB, 1, QLDS, ARG>(a, lds, di, st);
  case 2: return dense_with_depth<DT, KSB, 2, QLDS, ARG>(a, lds, di, st);
  case 3:
    if constexpr (QLDS || KSB * 3 <= 16) return dense_with_depth<DT, KSB, 3, QLDS, ARG>(a, lds, di, st);
    break;
  case 4:
    if constexpr (QLDS || KSB * 4 <= 16) return dense_with_depth<DT, KSB, 4, QLDS, ARG>(a, lds, di, st);
    break;
  }
  return MAXSIM_ERR_UNSUPPORTED;
}

template <int DT, bool QLDS, bool ARG>
int dense_by_ksb(int ksb, int qb, const DenseArgs &a, size_t lds, const DeviceInfo &di,
                 hipStream_t st) {
  switch (ksb) {
  case 1: return dense_by_qb<DT, 1, QLDS, ARG>(qb, a, lds, di, st);
  case 2: return dense_by_qb<DT, 2, QLDS, ARG>(qb, a, lds, di, st);
  case 3: return dense_by_qb<DT, 3, QLDS, ARG>(qb, a, lds, di, st);
  case 4: return dense_by_qb<DT, 4, QLDS, ARG>(qb, a, lds, di, st);
  case 5: return dense_by_qb<DT, 5, QLDS, ARG>(qb, a, lds, di, st);
  case 6: return dense_by_qb<DT, 6, QLDS, ARG>(qb, a, lds, di, st);
  case 7: return dense_by_qb<DT, 7, QLDS, ARG>(qb, a, lds, di, st);
  case 8: return dense_by_qb<DT, 8, QLDS, ARG>(qb, a, lds, di, st);
  }
  return MAXSIM_ERR_UNSUPPORTED;
}

template <int DT, bool ARG>
int dense_by_mode(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds, const DeviceInfo &di,
                  hipStream_t st) {
  return qlds ? dense_by_ksb<DT, true, ARG>(ksb, qb, a, lds, di, st)
              : dense_by_ksb<DT, false, ARG>(ksb, qb, a, lds, di, st);
}

}  // namespace
}  // namespace maxsim
