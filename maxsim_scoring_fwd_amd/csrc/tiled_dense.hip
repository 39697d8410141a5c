// Query-tiled kernels for bf16 / fp16 / fp32 storage (queries longer than 64 tokens).
#include "tiled_dispatch.hpp"

namespace maxsim {

int tiled_dense_run(const TiledArgs &a, int d, int dtype, const DeviceInfo &di, hipStream_t st) {
  const int ksb = d * elem_bytes(dtype) / 64;
  if (ksb != 1 && ksb != 2 && ksb != 4 && ksb != 8) return MAXSIM_ERR_UNSUPPORTED;
  if (tiled_tokens(a) > tiled_max_q(ksb)) return MAXSIM_ERR_UNSUPPORTED;
  const int tokens = tiled_tokens(a);
  // 16 waves of 4 query blocks each (measurement knob for the ColPali shape)
  static const int waves = env_knob("MAXSIM_TILED_WAVES", TILED_WAVES);
  if (waves == 16 && ksb == 4 && a.q_len > 768 && dtype == MAXSIM_BF16)
    return launch_tiled<DT_BF16, 4, 4, false, 16>(a, di, st);
  switch (dtype) {
  case MAXSIM_BF16: return tiled_by_ksb<DT_BF16, false>(ksb, tokens, a, di, st);
  case MAXSIM_FP16: return tiled_by_ksb<DT_FP16, false>(ksb, tokens, a, di, st);
  case MAXSIM_FP32: return tiled_by_ksb<DT_FP32, false>(ksb, tokens, a, di, st);
  }
  return MAXSIM_ERR_DTYPE;
}

}  // namespace maxsim
