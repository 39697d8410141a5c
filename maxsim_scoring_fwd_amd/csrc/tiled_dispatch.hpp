// Launch of the query-tiled kernel (long queries and INT8).
#pragma once

#include "host_common.hpp"
#include "tiled_kernel.hpp"

namespace maxsim {

// Query tokens of a launch: n_q queries, each padded to whole 16-token blocks.
inline int tiled_tokens(const TiledArgs &a) { return a.n_q * ((a.q_len + 15) & ~15); }

// Waves per workgroup. Every wave reads each A operand of a block from LDS and multiplies it
// by its QBW query blocks, so few blocks per wave leave the kernel bound by LDS reads, and with
// 8 waves a short query leaves some waves holding only padding. Up to 384 query tokens (within
// the register budget) run 4 waves of ceil(tokens / 64) blocks, two workgroups per CU; longer
// queries run 8 waves. INT8 rows of 64 bytes keep 8 waves (one thread per block row stages
// the per-token scales: 512 rows). Measured for INT8 with 100K documents of 128 tokens, 8
// against 4 waves, d = 128 / 256: 32 tokens 0.670 / 0.757 -> 0.506 / 0.556 ms, 128 tokens
// 0.589 / 0.796 -> 0.537 / 0.716 ms, 384 tokens 0.938 / 1.451 -> 0.915 / 1.314 ms.
inline int tiled_waves(int tokens, int ksb, bool i8) {
  const int qbw4 = (tokens + 63) / 64;
  return tokens <= 384 && qbw4 * ksb <= 32 && (!i8 || ksb >= 2) ? 4 : TILED_WAVES;
}

// Query blocks per wave for a number of query tokens (nw waves x 16 tokens x QBW >= tokens).
inline int tiled_qbw(int tokens, int nw) { return (tokens + nw * 16 - 1) / (nw * 16); }

// Largest query length the tiled kernel holds for KSB 64-byte chunks per row:
// the slice of one wave needs QBW * KSB * 4 VGPRs, kept at or below 128.
inline int tiled_max_q(int ksb) { return TILED_WAVES * 16 * (32 / ksb > 16 ? 16 : 32 / ksb); }

template <int DT, int KSB, int QBW, bool ARG, int NW = TILED_WAVES, bool BATCH = false>
int launch_tiled(const TiledArgs &a, const DeviceInfo &di, hipStream_t st) {
  auto kern = tiled_maxsim_kernel<DT, KSB, QBW, ARG, NW, BATCH>;
  const int bpc = blocks_per_cu((const void *)kern, NW * WAVE, 0);
  const int64_t max_wg = (int64_t)bpc * di.cus;
  int64_t grid = a.n_docs < max_wg ? a.n_docs : max_wg;
  if (grid < 1) grid = 1;
  char what[96];
  std::snprintf(what, sizeof what, "tiled<DT=%d,KSB=%d,QBW=%d,ARG=%d,NW=%d,BATCH=%d>", DT, KSB,
                QBW, (int)ARG, NW, (int)BATCH);
  log_launch(what, (const void *)kern, grid, NW * WAVE, 0, bpc);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * WAVE), 0, st, a);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

template <int DT, int KSB, bool ARG, bool BATCH, int NW>
int tiled_by_qbw(int qbw, const TiledArgs &a, const DeviceInfo &di, hipStream_t st) {
  switch (qbw) {
#define MAXSIM_TILED_CASE(N)                                                                      \
  case N:                                                                                         \
    if constexpr (N * KSB <= 32 && (NW == TILED_WAVES || N <= 6))                                 \
      return launch_tiled<DT, KSB, N, ARG, NW, BATCH>(a, di, st);                                 \
    break;
    MAXSIM_TILED_CASE(1)
    MAXSIM_TILED_CASE(2)
    MAXSIM_TILED_CASE(3)
    MAXSIM_TILED_CASE(4)
    MAXSIM_TILED_CASE(5)
    MAXSIM_TILED_CASE(6)
    MAXSIM_TILED_CASE(7)
    MAXSIM_TILED_CASE(8)
#undef MAXSIM_TILED_CASE
  }
  return MAXSIM_ERR_UNSUPPORTED;
}

template <int DT, int KSB, bool ARG, bool BATCH>
int tiled_by_waves(int tokens, const TiledArgs &a, const DeviceInfo &di, hipStream_t st) {
  const int nw = tiled_waves(tokens, KSB, DT == DT_I8);
  if constexpr (DT != DT_I8 || KSB >= 2) {
    if (nw == 4) return tiled_by_qbw<DT, KSB, ARG, BATCH, 4>(tiled_qbw(tokens, 4), a, di, st);
  }
  return tiled_by_qbw<DT, KSB, ARG, BATCH, TILED_WAVES>(tiled_qbw(tokens, TILED_WAVES), a, di, st);
}

// Launch for `tokens` query tokens (tiled_tokens) with KSB = ksb.
template <int DT, bool ARG, bool BATCH = false>
int tiled_by_ksb(int ksb, int tokens, const TiledArgs &a, const DeviceInfo &di, hipStream_t st) {
  switch (ksb) {
  case 1: return tiled_by_waves<DT, 1, ARG, BATCH>(tokens, a, di, st);
  case 2: return tiled_by_waves<DT, 2, ARG, BATCH>(tokens, a, di, st);
  case 4: return tiled_by_waves<DT, 4, ARG, BATCH>(tokens, a, di, st);
  case 8: return tiled_by_waves<DT, 8, ARG, BATCH>(tokens, a, di, st);
  }
  return MAXSIM_ERR_UNSUPPORTED;
}

// Dense storage (bf16 / fp16 / fp32) with q_len > 64; defined in tiled_dense.hip.
int tiled_dense_run(const TiledArgs &a, int d, int dtype, const DeviceInfo &di, hipStream_t st);
// The same, also writing per-token maxima and argmax; defined in tiled_dense_arg.hip.
int tiled_dense_argmax_run(const TiledArgs &a, int d, int dtype, const DeviceInfo &di,
                           hipStream_t st);
// Several queries (TiledArgs::n_q) in one pass, dense storage; defined in tiled_batch.hip.
int tiled_batch_run(const TiledArgs &a, int d, int dtype, const DeviceInfo &di, hipStream_t st);
// INT8 storage; defined in tiled_i8.hip.
int tiled_i8_run(const TiledArgs &a, int d, const DeviceInfo &di, hipStream_t st);

}  // namespace maxsim
