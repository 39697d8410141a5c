// Query-tiled kernels for bf16 / fp16 / fp32 storage (queries longer than 64 tokens).
#include "tiled_dispatch.hpp"

namespace maxsim {

int tiled_dense_run(const TiledArgs &a, int d, int dtype, const DeviceInfo &di, hipStream_t st) {
  const int ksb = d * elem_bytes(dtype) / 64;
  if (ksb != 1 && ksb != 2 && ksb != 4 && ksb != 8) return MAXSIM_ERR_UNSUPPORTED;
  if (tiled_tokens(a) > tiled_max_q(ksb)) return MAXSIM_ERR_UNSUPPORTED;
  const int tokens = tiled_tokens(a);
  switch (dtype) {
  case MAXSIM_BF16: return tiled_by_ksb<DT_BF16, false>(ksb, tokens, a, di, st);
  case MAXSIM_FP16: return tiled_by_ksb<DT_FP16, false>(ksb, tokens, a, di, st);
  case MAXSIM_FP32: return tiled_by_ksb<DT_FP32, false>(ksb, tokens, a, di, st);
  }
  return MAXSIM_ERR_DTYPE;
}

}  // namespace maxsim
