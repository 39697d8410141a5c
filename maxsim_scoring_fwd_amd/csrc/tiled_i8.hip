// Query-tiled kernels for INT8 x INT8 storage with per-token fp32 scales.
#include "tiled_dispatch.hpp"

namespace maxsim {

int tiled_i8_run(const TiledArgs &a, int d, const DeviceInfo &di, hipStream_t st) {
  const int ksb = d / 64;
  if (ksb != 1 && ksb != 2 && ksb != 4 && ksb != 8) return MAXSIM_ERR_UNSUPPORTED;
  if (tiled_tokens(a) > tiled_max_q(ksb)) return MAXSIM_ERR_UNSUPPORTED;
  const int tokens = tiled_tokens(a);
  if (a.tok_max) return tiled_by_ksb<DT_I8, true>(ksb, tokens, a, di, st);
  return tiled_by_ksb<DT_I8, false>(ksb, tokens, a, di, st);
}

}  // namespace maxsim
