// Streaming read, write and copy kernels and a matrix-core rate kernel used to
// calibrate measurements.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "../../include/maxsim_calib.h"
#include "device_common.hpp"
#include "host_common.hpp"

namespace {

using maxsim::u32x4_t;

constexpr int CAL_THREADS = 256;

// Each wave reads whole blocks of LOADS KiB: LOADS loads of 1 KiB in flight per wave,
// every load instruction covering 1 KiB of contiguous memory, the blocks dealt to the
// waves in turn.
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

// Each wave writes whole 16 KiB blocks with 128-bit stores (non-temporal with NT), every
// store instruction covering 1 KiB of contiguous memory (the pattern of a streaming writer).
template <bool NT>
__global__ void __launch_bounds__(CAL_THREADS) calib_write_kernel(u32x4_t *dst, size_t n16,
                                                                  uint32_t pattern, int contig) {
  constexpr size_t BLOCK16 = 64 * 16;
  const int lane = threadIdx.x & 63;
  const size_t wave = (size_t)blockIdx.x * (CAL_THREADS / 64) + (threadIdx.x >> 6);
  const size_t nwaves = (size_t)gridDim.x * (CAL_THREADS / 64);
  const size_t nblk = n16 / BLOCK16;
  const u32x4_t v = {pattern, pattern ^ 1u, pattern ^ 2u, pattern ^ 3u};
  // blocks dealt to the waves in turn, or with contig one contiguous range per wave
  size_t b0 = wave, b1 = nblk, bstep = nwaves;
  if (contig) {
    b0 = nblk * wave / nwaves;
    b1 = nblk * (wave + 1) / nwaves;
    bstep = 1;
  }
  for (size_t b = b0; b < b1; b += bstep) {
    u32x4_t *p = dst + b * BLOCK16 + lane;
#pragma unroll
    for (int u = 0; u < 16; u++) {
      if constexpr (NT)
        __builtin_nontemporal_store(v, p + u * 64);
      else
        p[u * 64] = v;
    }
  }
  for (size_t i = nblk * BLOCK16 + wave * 64 + lane; i < n16; i += nwaves * 64) dst[i] = v;
}

__global__ void __launch_bounds__(CAL_THREADS) calib_copy_kernel(const u32x4_t *src, u32x4_t *dst,
                                                                 size_t n16) {
  const size_t stride = (size_t)gridDim.x * CAL_THREADS;
  for (size_t i = (size_t)blockIdx.x * CAL_THREADS + threadIdx.x; i < n16; i += stride)
    dst[i] = src[i];
}

}  // namespace

extern "C" int maxsim_calib_read(const void *src, size_t bytes, int wgs_per_cu, uint32_t *sink,
                                 void *stream) {
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
  // 4 GiB on MI355X: one workgroup per CU (one wave per SIMD) 7.09 TB/s, two 6.94, as many
  // as fit (8) 6.82; fewer waves keep longer runs of each DRAM page open
  const int occ = maxsim::blocks_per_cu((const void *)kern, CAL_THREADS, 0);
  const int bpc = wgs_per_cu > 0 && wgs_per_cu < occ ? wgs_per_cu : occ;
  hipLaunchKernelGGL(kern, dim3(bpc * di.cus), dim3(CAL_THREADS), 0, (hipStream_t)stream,
                     (const u32x4_t *)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

extern "C" int maxsim_calib_write(void *dst, size_t bytes, int wgs_per_cu, int contig,
                                  void *stream) {
  if (!dst) return MAXSIM_ERR_NULL;
  if (bytes % 16 || !maxsim::aligned(dst, 16)) return MAXSIM_ERR_ALIGN;
  maxsim::DeviceInfo di;
  int rc = maxsim::current_device(di);
  if (rc != MAXSIM_OK) return rc;
  // 4 GiB on MI355X, ordinary 16-byte stores: one contiguous range per wave at two
  // workgroups per CU 5.86 TB/s, blocks in turn at one 5.58; non-temporal stores 5.03-5.47
  static const int nt = maxsim::env_knob("MAXSIM_CALIB_WRITE_NT", 0);
  auto kern = nt ? calib_write_kernel<true> : calib_write_kernel<false>;
  const int occ = maxsim::blocks_per_cu((const void *)kern, CAL_THREADS, 0);
  const int bpc = wgs_per_cu > 0 && wgs_per_cu < occ ? wgs_per_cu : occ;
  hipLaunchKernelGGL(kern, dim3(bpc * di.cus), dim3(CAL_THREADS), 0, (hipStream_t)stream,
                     (u32x4_t *)dst, bytes / 16, 0x3f800000u, contig);
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

// ---- matrix-core throughput: independent MFMA chains, no memory traffic ----

namespace {

using maxsim::f32x4_t;
using maxsim::i32x4_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int32_t i32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int MF_CHAINS = 8;

template <int KIND>
__global__ void __launch_bounds__(256) calib_mfma_kernel(int iters, float *sink) {
  const int lane = threadIdx.x & 63;
  u32x4_t a = {(uint32_t)lane, 1u, 2u, 3u}, b = {3u, (uint32_t)lane, 1u, 0x3f80u};
  if constexpr (KIND == 0 || KIND == 2) {
    // 16x16 output tiles
    typedef typename std::conditional<KIND == 0, f32x4_t, i32x4_t>::type acc_t;
    acc_t acc[MF_CHAINS] = {};
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int c = 0; c < MF_CHAINS; c++) {
        if constexpr (KIND == 0)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, b), acc[c], 0, 0, 0);
        else
          acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a),
                                                         __builtin_bit_cast(i32x4_t, b), acc[c], 0, 0, 0);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < MF_CHAINS; c++) s += (float)acc[c][0] + (float)acc[c][3];
    if (s == 1234.5f) sink[blockIdx.x] = s;  // keeps the chains alive
  } else {
    // 32x32 output tiles
    typedef typename std::conditional<KIND == 1, f32x16_t, i32x16_t>::type acc_t;
    acc_t acc[MF_CHAINS / 2] = {};
    for (int it = 0; it < iters; it++) {
#pragma unroll
      for (int c = 0; c < MF_CHAINS / 2; c++) {
        if constexpr (KIND == 1)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, b), acc[c], 0, 0, 0);
        else
          acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, a),
                                                         __builtin_bit_cast(i32x4_t, b), acc[c], 0, 0, 0);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < MF_CHAINS / 2; c++) s += (float)acc[c][0] + (float)acc[c][15];
    if (s == 1234.5f) sink[blockIdx.x] = s;
  }
}

}  // namespace

// kind 0: 16x16x32 bf16, 1: 32x32x16 bf16, 2: 16x16x64 i8, 3: 32x32x32 i8. Launches
// waves_per_simd x 4 x CUs waves of `iters` x 8 (16x16) or 4 (32x32) MFMAs each; returns
// the total FLOP / integer ops in *ops. sink: >= 65536 floats, never written in practice.
extern "C" int maxsim_calib_mfma(int kind, int iters, int waves_per_simd, float *sink,
                                 double *ops, void *stream) {
  if (!sink || !ops) return MAXSIM_ERR_NULL;
  if (kind < 0 || kind > 3 || iters < 1 || waves_per_simd < 1 || waves_per_simd > 8)
    return MAXSIM_ERR_SHAPE;
  maxsim::DeviceInfo di;
  int rc = maxsim::current_device(di);
  if (rc != MAXSIM_OK) return rc;
  const int grid = di.cus * waves_per_simd;  // 4 waves per workgroup = one per SIMD
  const double per = kind == 0 ? 16.0 * 16 * 32 * 2 : kind == 1 ? 32.0 * 32 * 16 * 2
                   : kind == 2 ? 16.0 * 16 * 64 * 2 : 32.0 * 32 * 32 * 2;
  const double per_iter = kind == 0 || kind == 2 ? 8 * per : 4 * per;
  *ops = per_iter * iters * grid * 4.0;
  hipStream_t st = (hipStream_t)stream;
  switch (kind) {
  case 0: hipLaunchKernelGGL(calib_mfma_kernel<0>, dim3(grid), dim3(256), 0, st, iters, sink); break;
  case 1: hipLaunchKernelGGL(calib_mfma_kernel<1>, dim3(grid), dim3(256), 0, st, iters, sink); break;
  case 2: hipLaunchKernelGGL(calib_mfma_kernel<2>, dim3(grid), dim3(256), 0, st, iters, sink); break;
  default: hipLaunchKernelGGL(calib_mfma_kernel<3>, dim3(grid), dim3(256), 0, st, iters, sink); break;
  }
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

// ---- vector-ALU throughput, matrix core + vector ALU together, LDS read rate ----

namespace {

constexpr int VA_CHAINS = 8;

// VALU: 8 independent chains of fp32 fused multiply-adds per lane (one VALU instruction
// each, never packed), `iters` rounds.
__global__ void __launch_bounds__(256) calib_valu_kernel(int iters, float *sink) {
  const int lane = threadIdx.x & 63;
  const float m = 1.0f + 1e-7f * lane, c = 1e-9f * (lane + 1);
  float x[VA_CHAINS];
#pragma unroll
  for (int j = 0; j < VA_CHAINS; j++) x[j] = 0.5f + 0.01f * j;
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < VA_CHAINS; j++) x[j] = __builtin_fmaf(x[j], m, c);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < VA_CHAINS; j++) s += x[j];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // keeps the chains alive
}

// Matrix core and vector ALU together: per round, 8 independent 16x16x64 int8 MFMA chains
// and V x 8 fp32 fused multiply-adds on 8 independent chains (no data flows between the
// two). With V = 0 it is the MFMA rate, and the time with V > 0 against the MFMA-only and
// VALU-only times tells how far the two units overlap.
template <int V>
__global__ void __launch_bounds__(256) calib_mix_kernel(int iters, float *sink) {
  const int lane = threadIdx.x & 63;
  const u32x4_t a = {(uint32_t)lane, 1u, 2u, 3u}, b = {3u, (uint32_t)lane, 1u, 0x01010101u};
  const float m = 1.0f + 1e-7f * lane, c = 1e-9f * (lane + 1);
  i32x4_t acc[MF_CHAINS] = {};
  float x[VA_CHAINS];
#pragma unroll
  for (int j = 0; j < VA_CHAINS; j++) x[j] = 0.5f + 0.01f * j;
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int ch = 0; ch < MF_CHAINS; ch++) {
      acc[ch] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a),
                                                      __builtin_bit_cast(i32x4_t, b), acc[ch], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < V; v++) x[(ch * V + v) % VA_CHAINS] = __builtin_fmaf(x[(ch * V + v) % VA_CHAINS], m, c);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int ch = 0; ch < MF_CHAINS; ch++) s += (float)acc[ch][0];
#pragma unroll
  for (int j = 0; j < VA_CHAINS; j++) s += x[j];
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

constexpr int LDS_THREADS = 1024;
constexpr int LDS_BYTES = 128 * 1024;  // the size of one PQ table slice: [16][256][8] fp32

// LDS read rate: every lane issues 16-byte reads. Pattern 0: a wave reads 1 KiB of
// contiguous LDS (conflict-free). Pattern 1: the PQ lookup pattern: lane pairs share a
// token, each lane reads the 16 bytes of its half of table row (m, code) of a [16][256][8]
// fp32 table; each token has 16 random codes (a hash of its index), and every round XORs
// them with a round-dependent byte (a bijection on codes, so they stay uniform and their
// collisions change from round to round).
template <int PATTERN>
__global__ void __launch_bounds__(LDS_THREADS) calib_lds_kernel(int iters, uint32_t *sink) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  for (int i = threadIdx.x; i < LDS_BYTES / 16; i += LDS_THREADS)
    reinterpret_cast<u32x4_t *>(lds)[i] = u32x4_t{(uint32_t)i, (uint32_t)i * 3u, 7u, 1u};
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t code[16];
  uint32_t h = (uint32_t)(threadIdx.x >> 1) * 0x9E3779B9u + blockIdx.x * 0x85EBCA6Bu + 1u;
#pragma unroll
  for (int m = 0; m < 16; m++) {
    h ^= h << 13;
    h ^= h >> 17;
    h ^= h << 5;
    code[m] = h >> 24;
  }
  uint32_t acc = 0;
  for (int it = 0; it < iters; it++) {
    const uint32_t r = ((uint32_t)it * 0x9E3779B9u) >> 24;  // the same in every lane
#pragma unroll
    for (int m = 0; m < 16; m++) {
      uint32_t off;
      if constexpr (PATTERN == 0)
        off = ((uint32_t)(w * 16 + m) * 1024u + (uint32_t)it * 16384u + lane * 16u) % LDS_BYTES;
      else
        off = ((uint32_t)m * 256u + (code[m] ^ r)) * 32u + (lane & 1) * 16u;
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(lds + off);
      acc ^= v[0] + v[3];
    }
  }
  if (acc == 0x12345678u) sink[blockIdx.x] = acc;
}

}  // namespace

// Launches waves_per_simd x 4 x CUs waves of `iters` x 8 fused multiply-adds per lane;
// *ops receives the FLOP count (2 per lane per FMA).
extern "C" int maxsim_calib_valu(int iters, int waves_per_simd, float *sink, double *ops,
                                 void *stream) {
  if (!sink || !ops) return MAXSIM_ERR_NULL;
  if (iters < 1 || waves_per_simd < 1 || waves_per_simd > 8) return MAXSIM_ERR_SHAPE;
  maxsim::DeviceInfo di;
  int rc = maxsim::current_device(di);
  if (rc != MAXSIM_OK) return rc;
  const int grid = di.cus * waves_per_simd;
  *ops = 2.0 * 64 * VA_CHAINS * (double)iters * grid * 4.0;
  hipLaunchKernelGGL(calib_valu_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

// valu_per_mfma in {0, 1, 2, 4, 8}; *ops receives the launch's int8 MFMA integer ops.
extern "C" int maxsim_calib_mix(int valu_per_mfma, int iters, int waves_per_simd, float *sink,
                                double *ops, void *stream) {
  if (!sink || !ops) return MAXSIM_ERR_NULL;
  const int V = valu_per_mfma;
  if (iters < 1 || waves_per_simd < 1 || waves_per_simd > 8 ||
      (V != 0 && V != 1 && V != 2 && V != 4 && V != 8))
    return MAXSIM_ERR_SHAPE;
  maxsim::DeviceInfo di;
  int rc = maxsim::current_device(di);
  if (rc != MAXSIM_OK) return rc;
  const int grid = di.cus * waves_per_simd;
  *ops = 16.0 * 16 * 64 * 2 * MF_CHAINS * (double)iters * grid * 4.0;
  hipStream_t st = (hipStream_t)stream;
  switch (V) {
  case 0: hipLaunchKernelGGL(calib_mix_kernel<0>, dim3(grid), dim3(256), 0, st, iters, sink); break;
  case 1: hipLaunchKernelGGL(calib_mix_kernel<1>, dim3(grid), dim3(256), 0, st, iters, sink); break;
  case 2: hipLaunchKernelGGL(calib_mix_kernel<2>, dim3(grid), dim3(256), 0, st, iters, sink); break;
  case 4: hipLaunchKernelGGL(calib_mix_kernel<4>, dim3(grid), dim3(256), 0, st, iters, sink); break;
  default: hipLaunchKernelGGL(calib_mix_kernel<8>, dim3(grid), dim3(256), 0, st, iters, sink); break;
  }
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

// One 1024-thread workgroup per CU with 128 KiB of LDS; *bytes receives the LDS bytes read.
extern "C" int maxsim_calib_lds(int pattern, int iters, uint32_t *sink, double *bytes,
                                void *stream) {
  if (!sink || !bytes) return MAXSIM_ERR_NULL;
  if ((pattern != 0 && pattern != 1) || iters < 1) return MAXSIM_ERR_SHAPE;
  maxsim::DeviceInfo di;
  int rc = maxsim::current_device(di);
  if (rc != MAXSIM_OK) return rc;
  if (di.max_lds < (size_t)LDS_BYTES) return MAXSIM_ERR_UNSUPPORTED;
  auto kern = pattern == 0 ? calib_lds_kernel<0> : calib_lds_kernel<1>;
  *bytes = 16.0 * 16 * (double)iters * LDS_THREADS * di.cus;
  hipLaunchKernelGGL(kern, dim3(di.cus), dim3(LDS_THREADS), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}
