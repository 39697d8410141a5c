// Host-side helpers of libmaxsim: argument checks, device checks, launch sizing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "../../include/maxsim.h"

namespace maxsim {

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline int elem_bytes(int dtype) {
  switch (dtype) {
  case MAXSIM_BF16:
  case MAXSIM_FP16: return 2;
  case MAXSIM_FP32: return 4;
  default: return 0;
  }
}

// Checks shared by the dense entry points; pure host logic, no HIP calls.
inline int check_dense(const void *Q, int q_len, const void *D, int64_t n_docs, int d, int dtype,
                       const float *out) {
  if (elem_bytes(dtype) == 0) return MAXSIM_ERR_DTYPE;
  if (n_docs < 0 || q_len < 1 || q_len > MAXSIM_MAX_Q_LEN) return MAXSIM_ERR_SHAPE;
  if (d < MAXSIM_MIN_D || d > MAXSIM_MAX_D || d % 32 != 0) return MAXSIM_ERR_SHAPE;
  if (!Q || !D || !out) return MAXSIM_ERR_NULL;
  if (!aligned(Q, 16) || !aligned(D, 16) || !aligned(out, 4)) return MAXSIM_ERR_ALIGN;
  return MAXSIM_OK;
}

struct DeviceInfo {
  int ok = 0;   // gfx950 present and current
  int cus = 0;  // compute units
  size_t max_lds = 0;
};

// Properties of the current device, cached per device ordinal.
inline int current_device(DeviceInfo &info) {
  static std::mutex mu;
  static std::unordered_map<int, DeviceInfo> cache;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MAXSIM_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    DeviceInfo di;
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess) {
      di.ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
      di.cus = p.multiProcessorCount;
      di.max_lds = p.sharedMemPerBlock;
    }
    it = cache.emplace(dev, di).first;
  }
  info = it->second;
  return info.ok ? MAXSIM_OK : MAXSIM_ERR_DEVICE;
}

// Resident workgroups per CU for a kernel at a block size and LDS size (cached).
inline int blocks_per_cu(const void *kernel, int threads, size_t lds) {
  static std::mutex mu;
  static std::unordered_map<uint64_t, int> cache;
  const uint64_t key = (uint64_t)(uintptr_t)kernel ^ ((uint64_t)lds << 40) ^ ((uint64_t)threads << 56);
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess || n < 1)
    n = 1;
  cache.emplace(key, n);
  return n;
}

// Integer knob from the environment (read once per name); used to force a kernel variant
// for A/B measurements.
inline int env_knob(const char *name, int dflt) {
  const char *v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

// MAXSIM_LOG_LAUNCH=1: one line on stderr per launch of the scoring kernels (variant, grid,
// workgroup, LDS, resident workgroups per CU and the kernel's register counts), for checking
// launch sizing against the hardware's limits.
inline void log_launch(const char *what, const void *kernel, int64_t grid, int threads,
                       size_t lds, int bpc) {
  static const int on = env_knob("MAXSIM_LOG_LAUNCH", 0);
  if (!on) return;
  hipFuncAttributes fa{};
  const bool ok = hipFuncGetAttributes(&fa, kernel) == hipSuccess;
  std::fprintf(stderr,
               "maxsim launch: %s grid=%lld threads=%d dyn_lds=%zu static_lds=%zu "
               "blocks_per_cu=%d regs=%d max_threads=%d\n",
               what, (long long)grid, threads, lds, ok ? (size_t)fa.sharedSizeBytes : (size_t)0,
               bpc, ok ? fa.numRegs : -1, ok ? fa.maxThreadsPerBlock : -1);
}

}  // namespace maxsim
