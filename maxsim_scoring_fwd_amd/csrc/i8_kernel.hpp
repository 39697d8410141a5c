// INT8 x INT8 MaxSim kernel (placeholder until the kernel lands).
#pragma once

#include "device_common.hpp"
#include "host_common.hpp"

namespace maxsim {

struct I8Args {
  const int8_t *Q;
  const float *q_scale;
  int q_len;
  const int8_t *D;
  const float *d_scale;
  const int64_t *offsets;
  int64_t n_docs;
  int nd;
  int d;
  float *out;
  float *tok_max;
  int32_t *tok_arg;
};

inline int i8_run(const I8Args &, const DeviceInfo &, hipStream_t) { return MAXSIM_ERR_UNSUPPORTED; }

}  // namespace maxsim
