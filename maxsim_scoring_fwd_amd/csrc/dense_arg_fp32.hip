// Dense MaxSim kernels with per-token maxima and argmax, fp32 storage.
#include "dense_variants.hpp"

namespace maxsim {

int dense_argmax_dispatch_fp32(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds,
                               const DeviceInfo &di, hipStream_t st) {
  return dense_by_mode<DT_FP32, true>(qlds, ksb, qb, a, lds, di, st);
}

}  // namespace maxsim
