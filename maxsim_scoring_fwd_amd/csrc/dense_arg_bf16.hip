// Dense MaxSim kernels with per-token maxima and argmax, bf16 storage.
#include "dense_variants.hpp"

namespace maxsim {

int dense_argmax_dispatch_bf16(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds,
                               const DeviceInfo &di, hipStream_t st) {
  return dense_by_mode<DT_BF16, true>(qlds, ksb, qb, a, lds, di, st);
}

}  // namespace maxsim
