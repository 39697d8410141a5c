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

// INT8 storage: int32 dot products on the matrix core, per-token fp32 scales applied
// before the max (Flash-MaxSim abstract: INT8 x INT8 scoring).
constexpr int DT_I8 = 3;
template <> struct Elem<DT_I8> { static constexpr int bytes = 1; };

// 16x16x64 i8 -> i32, K = 64 int8 = one 64-byte chunk per row (the chunk layout below).
__device__ __forceinline__ i32x4_t chunk_mfma_i8(u32x4_t a, u32x4_t b, i32x4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a),
                                               __builtin_bit_cast(i32x4_t, b), c, 0, 0, 0);
}

// INT8 scale products on the matrix core. Four 16x16 blocks, K = 1: block k of the result,
// lane l, element 4k + r, is a * b of lane (16k + 4 * (l / 16) + r) of the A operand and lane
// (16k + l % 16) of the B operand: with A = a tile's 16 document-token scales (lane l: row
// l % 16, the same in every block) and B = the scales of four query blocks (lane l: block
// l / 16, column l % 16), element 4k + r of lane l is the scale product of accumulator
// element r of query block k in that lane. One product plus zero per entry, rounded once:
// fl32(q_scale * d_scale), bit for bit the rounded multiply.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16_t scale_products(float a, float b) {
  const f32x16_t zero = {};
  return __builtin_amdgcn_mfma_f32_16x16x1f32(a, b, zero, 0, 0, 0);
}

// Accumulator of one 16x16 tile: fp32, or int32 for INT8.
template <bool INT> struct AccType { using type = f32x4_t; };
template <> struct AccType<true> { using type = i32x4_t; };

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

// ---- reductions across lanes, in registers (no LDS round trip) ----
// A 16x16 accumulator spreads one column over the four 16-lane row groups of the wave
// (lanes c, c + 16, c + 32, c + 48), and the 16 columns of a row group are its 16 lanes.

// Both members of each pair of row groups, in every lane of the pair: gfx950's
// v_permlane16_swap exchanges rows 1 and 3 of its first operand with rows 0 and 2 of its
// second; given the same value twice it returns, in each lane, the lane's own value and
// the one of lane ^ 16 (in some order). v_permlane32_swap does the same for lane ^ 32.
template <int XOR> __device__ __forceinline__ void row_pair(uint32_t x, uint32_t &p0, uint32_t &p1) {
  static_assert(XOR == 16 || XOR == 32, "row groups pair at distance 16 or 32");
  if constexpr (XOR == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    p0 = p[0];
    p1 = p[1];
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    p0 = p[0];
    p1 = p[1];
  }
}

// s plus the s of lane ^ XOR (XOR 16 or 32), in every lane: both lanes of a pair get the
// same sum (their two terms in either order, and double addition commutes exactly).
template <int XOR> __device__ __forceinline__ double pair_sum_f64(double s) {
  const uint64_t u = __builtin_bit_cast(uint64_t, s);
  uint32_t l0, l1, h0, h1;
  row_pair<XOR>((uint32_t)u, l0, l1);
  row_pair<XOR>((uint32_t)(u >> 32), h0, h1);
  return __builtin_bit_cast(double, ((uint64_t)h0 << 32) | l0) +
         __builtin_bit_cast(double, ((uint64_t)h1 << 32) | l1);
}

// Maximum over the four row groups, in every lane.
__device__ __forceinline__ float max_row_groups(float v) {
  uint32_t a, b;
  row_pair<16>(__float_as_uint(v), a, b);
  v = __builtin_fmaxf(__uint_as_float(a), __uint_as_float(b));
  row_pair<32>(__float_as_uint(v), a, b);
  return __builtin_fmaxf(__uint_as_float(a), __uint_as_float(b));
}

// (value, index) with the largest value over the four row groups, equal values keeping
// the lower index, in every lane. The choice is symmetric in the two members of a pair.
__device__ __forceinline__ void argmax_row_groups(float &v, int &j) {
  uint32_t va, vb, ja, jb;
  row_pair<16>(__float_as_uint(v), va, vb);
  row_pair<16>((uint32_t)j, ja, jb);
  bool take_b = __uint_as_float(vb) > __uint_as_float(va) ||
                (__uint_as_float(vb) == __uint_as_float(va) && (int)jb < (int)ja);
  v = __uint_as_float(take_b ? vb : va);
  j = (int)(take_b ? jb : ja);
  row_pair<32>(__float_as_uint(v), va, vb);
  row_pair<32>((uint32_t)j, ja, jb);
  take_b = __uint_as_float(vb) > __uint_as_float(va) ||
           (__uint_as_float(vb) == __uint_as_float(va) && (int)jb < (int)ja);
  v = __uint_as_float(take_b ? vb : va);
  j = (int)(take_b ? jb : ja);
}

// DPP row permutes (within each 16-lane row): lane ^ 1, lane ^ 2, 7 - lane within each
// half row, 15 - lane within the row.
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141; // row_half_mirror
constexpr int DPP_MIRROR = 0x140;      // row_mirror

template <int CTRL> __device__ __forceinline__ float dpp_f32(float x) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL> __device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, CTRL, 0xF, 0xF, true);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum over the 16 lanes of each row group, in every lane of it. The pairs are those of
// a butterfly over lane ^ 1, ^ 2, ^ 4, ^ 8 (after the first two steps a quad holds one
// value, so the mirrors pair whole quads, then whole half rows).
template <typename T> __device__ __forceinline__ T sum_row16(T s) {
  if constexpr (sizeof(T) == 8) {
    s += dpp_f64<DPP_XOR1>(s);
    s += dpp_f64<DPP_XOR2>(s);
    s += dpp_f64<DPP_HALF_MIRROR>(s);
    s += dpp_f64<DPP_MIRROR>(s);
  } else {
    s += dpp_f32<DPP_XOR1>(s);
    s += dpp_f32<DPP_XOR2>(s);
    s += dpp_f32<DPP_HALF_MIRROR>(s);
    s += dpp_f32<DPP_MIRROR>(s);
  }
  return s;
}

}  // namespace maxsim
