// Device helpers shared by the MaxSim kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace maxsim {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

enum { DT_BF16 = 0, DT_FP16 = 1, DT_FP32 = 2 };

constexpr int WAVE = 64;

template <int DT> struct Elem;
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_FP16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_FP32> { static constexpr int bytes = 4; };

// One "chunk" = 16 bytes per lane, 64 lanes: 16 rows x 64 contiguous bytes.
// Lane l holds row (l % 16) and bytes [16*(l/16), 16*(l/16)+16) of the row's
// 64-byte piece. chunk_mfma folds one chunk of the doc tile (operand A, rows =
// document tokens) against the matching chunk of 16 query tokens (operand B,
// columns = query tokens) into the 16x16 fp32 accumulator. The same byte
// slice of a row feeds the same k slot of A and B, so the dot product over the
// chunk's elements is exact whatever order the matrix core uses internally.
//
// 16x16 accumulator layout: lane l holds column (l % 16) and rows
// 4*(l/16) .. 4*(l/16)+3 in elements 0..3.
template <int DT> struct ChunkMfma;

template <> struct ChunkMfma<DT_BF16> {
  static constexpr int mfmas = 1;  // 16x16x32: K = 32 bf16 = 64 bytes per row
  __device__ __forceinline__ static f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

template <> struct ChunkMfma<DT_FP16> {
  static constexpr int mfmas = 1;  // 16x16x32 f16
  __device__ __forceinline__ static f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

template <> struct ChunkMfma<DT_FP32> {
  static constexpr int mfmas = 4;  // 4 x 16x16x4 f32: K = 16 floats = 64 bytes per row
  __device__ __forceinline__ static f32x4_t run(u32x4_t a, u32x4_t b, f32x4_t c) {
    // Elements are copied to scalars first: a bit cast of a vector-element subscript
    // would read the vector's first element.
    const uint32_t a0 = a.x, a1 = a.y, a2 = a.z, a3 = a.w;
    const uint32_t b0 = b.x, b1 = b.y, b2 = b.z, b3 = b.w;
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a0), __uint_as_float(b0), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a1), __uint_as_float(b1), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a2), __uint_as_float(b2), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a3), __uint_as_float(b3), c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ int64_t uniform(int64_t v) {
  uint64_t u = (uint64_t)v;
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ u32x4_t load16(const char *p) {
  return *reinterpret_cast<const u32x4_t *>(p);
}

// Streaming load: the data is read exactly once, so it is marked non-temporal.
__device__ __forceinline__ u32x4_t load16_nt(const char *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

// Order the wave's LDS accesses before and after this point (a wave-level barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float max4(f32x4_t v) {
  return __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), __builtin_fmaxf(v[2], v[3]));
}

}  // namespace maxsim
