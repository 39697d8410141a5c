// Dense MaxSim kernels for INT8 storage with per-token scales: queries of up to 64 tokens,
// rows of 64, 128 or 256 bytes (d = 64, 128, 256), the query in registers.
#include "dense_variants.hpp"

namespace maxsim {

namespace {

template <bool ARG>
int dense_i8_by_ksb(int ksb, int qb, const DenseArgs &a, const DeviceInfo &di, hipStream_t st) {
  switch (ksb) {
  case 1: return dense_by_qb<DT_I8, 1, false, ARG>(qb, a, 0, di, st);
  case 2: return dense_by_qb<DT_I8, 2, false, ARG>(qb, a, 0, di, st);
  case 4: return dense_by_qb<DT_I8, 4, false, ARG>(qb, a, 0, di, st);
  }
  return MAXSIM_ERR_UNSUPPORTED;
}

}  // namespace

int dense_i8_run(int ksb, int qb, const DenseArgs &a, const DeviceInfo &di, hipStream_t st) {
  return a.tok_max ? dense_i8_by_ksb<true>(ksb, qb, a, di, st)
                   : dense_i8_by_ksb<false>(ksb, qb, a, di, st);
}

}  // namespace maxsim
