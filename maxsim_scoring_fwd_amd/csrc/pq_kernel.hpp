// PQ table and lookup-scoring kernels (placeholder until the kernels land).
#pragma once

#include "device_common.hpp"
#include "host_common.hpp"

namespace maxsim {

constexpr int PQ_MAX_Q = 64;

struct PqTableArgs {
  const char *Q;
  int q_len;
  int dtype;
  const float *C;
  int M, K, dsub;
  float *T;
};

struct PqScoreArgs {
  const float *T;
  int q_len;
  const uint8_t *codes;
  const int64_t *offsets;
  int64_t n_docs;
  int nd;
  float *out;
};

inline int pq_tables_run(const PqTableArgs &, const DeviceInfo &, hipStream_t) {
  return MAXSIM_ERR_UNSUPPORTED;
}
inline int pq_score_run(const PqScoreArgs &, const DeviceInfo &, hipStream_t) {
  return MAXSIM_ERR_UNSUPPORTED;
}

}  // namespace maxsim
