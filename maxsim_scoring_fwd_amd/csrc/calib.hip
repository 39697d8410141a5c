// Streaming read and copy kernels used to calibrate bandwidth measurements.
#include <hip/hip_runtime.h>

#include "../../include/maxsim_calib.h"
#include "device_common.hpp"
#include "host_common.hpp"

namespace {

using maxsim::u32x4_t;

constexpr int CAL_THREADS = 256;

// Each wave reads whole blocks of LOADS KiB: LOADS loads of 1 KiB in flight per wave,
// every load instruction covering 1 KiB of contiguous memory.
template <bool NT, int LOADS>
__global__ void __launch_bounds__(CAL_THREADS) calib_read_kernel(const u32x4_t *src, size_t n16,
                                                                 uint32_t *sink) {
  constexpr int CAL_LOADS = LOADS;
  constexpr size_t CAL_BLOCK16 = 64 * CAL_LOADS;  // 16-byte pieces per block
  const int lane = threadIdx.x & 63;
  const size_t wave = (size_t)blockIdx.x * (CAL_THREADS / 64) + (threadIdx.x >> 6);
  const size_t nwaves = (size_t)gridDim.x * (CAL_THREADS / 64);
  const size_t nblk = n16 / CAL_BLOCK16;
  uint32_t acc = 0;
  for (size_t b = wave; b < nblk; b += nwaves) {
    const u32x4_t *p = src + b * CAL_BLOCK16 + lane;
    u32x4_t v[CAL_LOADS];
#pragma unroll
    for (int u = 0; u < CAL_LOADS; u++) v[u] = NT ? __builtin_nontemporal_load(p + u * 64) : p[u * 64];
#pragma unroll
    for (int u = 0; u < CAL_LOADS; u++) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // tail pieces past the last whole block
  for (size_t i = nblk * CAL_BLOCK16 + wave * 64 + lane; i < n16; i += nwaves * 64) {
    u32x4_t v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  acc = __reduce_xor_sync(~0ull, acc);
  if (lane == 0) atomicXor(&sink[blockIdx.x & 65535], acc);
}

__global__ void __launch_bounds__(CAL_THREADS) calib_copy_kernel(const u32x4_t *src, u32x4_t *dst,
                                                                 size_t n16) {
  const size_t stride = (size_t)gridDim.x * CAL_THREADS;
  for (size_t i = (size_t)blockIdx.x * CAL_THREADS + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

}  // namespace

extern "C" int maxsim_calib_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (!src || !sink) return MAXSIM_ERR_NULL;
  if (bytes % 16 || !maxsim::aligned(src, 16)) return MAXSIM_ERR_ALIGN;
  maxsim::DeviceInfo di;
  int rc = maxsim::current_device(di);
  if (rc != MAXSIM_OK) return rc;
  static const int nt = maxsim::env_knob("MAXSIM_CALIB_NT", 1);
  static const int loads = maxsim::env_knob("MAXSIM_CALIB_LOADS", 16);
  auto kern = nt ? calib_read_kernel<true, 16> : calib_read_kernel<false, 16>;
  if (loads == 8) kern = nt ? calib_read_kernel<true, 8> : calib_read_kernel<false, 8>;
  if (loads == 32) kern = nt ? calib_read_kernel<true, 32> : calib_read_kernel<false, 32>;
  const int bpc = maxsim::blocks_per_cu((const void *)kern, CAL_THREADS, 0);
  hipLaunchKernelGGL(kern, dim3(bpc * di.cus), dim3(CAL_THREADS), 0, (hipStream_t)stream,
                     (const u32x4_t *)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

extern "C" int maxsim_calib_copy(const void *src, void *dst, size_t bytes, void *stream) {
  if (!src || !dst) return MAXSIM_ERR_NULL;
  if (bytes % 16 || !maxsim::aligned(src, 16) || !maxsim::aligned(dst, 16)) return MAXSIM_ERR_ALIGN;
  maxsim::DeviceInfo di;
  int rc = maxsim::current_device(di);
  if (rc != MAXSIM_OK) return rc;
  const int bpc = maxsim::blocks_per_cu((const void *)calib_copy_kernel, CAL_THREADS, 0);
  hipLaunchKernelGGL(calib_copy_kernel, dim3(bpc * di.cus), dim3(CAL_THREADS), 0,
                     (hipStream_t)stream, (const u32x4_t *)src, (u32x4_t *)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}
