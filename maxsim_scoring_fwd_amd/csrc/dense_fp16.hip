// Dense MaxSim kernels for fp16 storage.
#include "dense_variants.hpp"

namespace maxsim {

int dense_dispatch_fp16(bool qlds, int ksb, int qb, const DenseArgs &a, size_t lds,
                        const DeviceInfo &di, hipStream_t st) {
  return dense_by_mode<DT_FP16, false>(qlds, ksb, qb, a, lds, di, st);
}

}  // namespace maxsim
