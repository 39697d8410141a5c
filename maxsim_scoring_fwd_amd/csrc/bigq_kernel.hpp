// Long-query dense MaxSim (q_len > 64): placeholder until the kernel lands.
#pragma once

#include "dense_kernel.hpp"
#include "host_common.hpp"

namespace maxsim {

inline int dense_big_q_run(const DenseArgs &, int, int, const DeviceInfo &, hipStream_t) {
  return MAXSIM_ERR_UNSUPPORTED;
}

}  // namespace maxsim
