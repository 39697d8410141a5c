// Top-k selection over the scores: the k best documents of each row of scores, ordered by
// score (descending), ties by document index (ascending).
//
// What it computes (the stage after scoring in late-interaction retrieval: TileMaxSim deep
// reading, sections 4 and 6 — the documents handed on are the best-scoring ones): for a row
// of n fp32 scores, the k entries that come first in the order (score descending, index
// ascending), in that order.
//
// Every candidate is one 64-bit key: the score mapped to an unsigned integer whose order is
// the reverse of the float order (a smaller key is a better score; -0 and +0 map to the same
// key) in the high half, the document index in the low half. One unsigned comparison then
// implements the whole order, ties included, so the result is exact and the same on every
// run. The reported score is read back from the score row by index (its exact bits).
//
// k <= 128: sorted runs held by waves (bitonic top-k).
//  * A run is 128 keys in ascending order held by one wave, two per lane (positions 2l and
//    2l + 1 in lane l). A wave sorts its run with a bitonic network whose exchanges between
//    lanes are vector-unit moves (DPP row and quad permutes, v_permlane16/32_swap): no LDS
//    traffic and no barriers.
//  * Two runs merge into the best 128 of their union: the elementwise minimum of one run and
//    the other reversed is bitonic and holds those 128 keys; seven half-cleaner steps sort it.
//  * Pass 1: a workgroup of 16 waves takes 2048 scores, each wave sorts 128 of them, and the
//    16 runs merge in a tree through LDS (four barriers) into the chunk's best 128.
//  * Later passes: a workgroup merges up to 64 runs (four per wave, loaded at once, then the
//    tree). The top-100 of 100K scores is one pass of 49 workgroups and one merge of 49 runs.
//    Two launches: each launch boundary costs about 7 us here, and merging across
//    workgroups within one launch (device-scope fences on every workgroup) measured slower.
// 128 < k <= 1024: a workgroup sorts 2048 keys in LDS (bitonic) and keeps k, level by level
// until one chunk remains.
// No atomics anywhere. Rows (queries of a batch) are independent: blockIdx.y is the row.
#pragma once

#include "device_common.hpp"

namespace maxsim {

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_CHUNK = 2 * TOPK_THREADS;  // keys sorted per workgroup
constexpr int TOPK_MAX_K = TOPK_THREADS;      // at most half a chunk survives a level

// fp32 score -> unsigned key, smaller for better scores (-inf last; NaN is not ordered).
// -0 and +0 compare equal as scores, so both get +0's key and the index decides.
__device__ __forceinline__ uint32_t topk_score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  const uint32_t ascending = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~ascending;
}

struct TopkLevelArgs {
  const float *scores;      // level 1: [rows][n] scores (else nullptr)
  const uint64_t *in_keys;  // later levels: [rows][count] keys
  int64_t count;            // entries per row at this level
  int64_t in_stride;        // elements between rows of the input
  int k;                    // entries kept per chunk
  uint64_t *out_keys;       // [rows][chunks * k], or nullptr on the final level
  int64_t out_stride;
  float *out_scores;        // final level: [rows][k]
  int32_t *out_index;       // final level: [rows][k]
  const float *orig;        // the score rows [rows][n]: reported scores are read back by index
  int64_t n;
};

__global__ void __launch_bounds__(TOPK_THREADS) topk_level_kernel(TopkLevelArgs a) {
  __shared__ uint64_t key[TOPK_CHUNK];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * TOPK_CHUNK;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int e = t + h * TOPK_THREADS;
    const int64_t i = c0 + e;
    uint64_t v = ~0ull;  // padding sorts last
    if (i < a.count) {
      if (a.scores)
        v = ((uint64_t)topk_score_key(a.scores[row * a.in_stride + i]) << 32) | (uint64_t)i;
      else
        v = a.in_keys[row * a.in_stride + i];
    }
    key[e] = v;
  }
  // bitonic sort, ascending: each thread owns one compare-exchange pair per step. A pair
  // with stride < 2 * WAVE lies within the 2 * WAVE keys of the thread's own wave. Between
  // two steps a workgroup barrier is needed only if one of them crosses waves (reads or
  // writes keys of other waves); otherwise the wave's own LDS order suffices.
  bool prev_cross = true;  // the keys were just written by other threads
  for (int size = 2; size <= TOPK_CHUNK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const bool cross = stride >= 2 * WAVE;
      if (cross || prev_cross)
        __syncthreads();
      else
        wave_lds_sync();
      prev_cross = cross;
      const int lo = 2 * t - (t & (stride - 1));  // first index of this thread's pair
      const int hi = lo + stride;
      const bool up = (lo & size) == 0;
      const uint64_t x = key[lo], y = key[hi];
      if ((x > y) == up) {
        key[lo] = y;
        key[hi] = x;
      }
    }
  }
  __syncthreads();
  const int keep = a.k;
  for (int e = t; e < keep; e += TOPK_THREADS) {
    const uint64_t v = key[e];
    if (a.out_keys) {
      a.out_keys[row * a.out_stride + (int64_t)blockIdx.x * keep + e] = v;
    } else {
      const bool real = v != ~0ull;
      const uint32_t idx = (uint32_t)v;
      a.out_scores[row * keep + e] = real ? a.orig[row * a.n + idx] : -__builtin_inff();
      a.out_index[row * keep + e] = real ? (int32_t)idx : -1;
    }
  }
}


// ---------------------------------------------------------------- k <= 128: sorted runs

constexpr int RUN = 128;                      // keys per run: one wave, two per lane
constexpr int RUN_WAVES = 16;
constexpr int RUN_THREADS = RUN_WAVES * WAVE;
constexpr int RUN_CHUNK = RUN_WAVES * RUN;    // scores per workgroup of the first pass
constexpr int RUN_FANIN = 4 * RUN_WAVES;      // runs merged per workgroup of later passes
constexpr int RUN_MAX_K = RUN;

// The value of lane (lane ^ M), M < 64, by vector-unit moves only (no LDS round trip):
// quad permutes for lane ^ 1, ^ 2, ^ 3, row_half_mirror (^ 7), row_ror:8 (^ 8 within a row
// of 16), row_mirror (^ 15), v_permlane16_swap (^ 16), v_permlane32_swap (^ 32), and their
// compositions: ^ 4 = (^ 7)(^ 3), ^ 31 = (^ 15)(^ 16), ^ 63 = (^ 31)(^ 32). Other masks take
// ds_swizzle (xor within 32 lanes).
template <int M> __device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  static_assert(M > 0 && M < 64, "a lane of the wave");
  if constexpr (M == 1) {
    return __builtin_amdgcn_update_dpp(0u, x, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_update_dpp(0u, x, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 3) {
    return __builtin_amdgcn_update_dpp(0u, x, 0x1B, 0xF, 0xF, true);  // quad_perm [3,2,1,0]
  } else if constexpr (M == 4) {
    return lane_xor<3>(lane_xor<7>(x));
  } else if constexpr (M == 7) {
    return __builtin_amdgcn_update_dpp(0u, x, 0x141, 0xF, 0xF, true);  // row_half_mirror
  } else if constexpr (M == 8) {
    return __builtin_amdgcn_update_dpp(0u, x, 0x128, 0xF, 0xF, true);  // row_ror:8
  } else if constexpr (M == 15) {
    return __builtin_amdgcn_update_dpp(0u, x, 0x140, 0xF, 0xF, true);  // row_mirror
  } else if constexpr (M == 16 || M == 32) {
    // with x in both operands, the first result holds in the upper member of each pair of
    // 16- (32-) lane groups the lower member's value, the second result the reverse
    const auto p = M == 16 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                           : __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (threadIdx.x & M) ? p[0] : p[1];
  } else if constexpr (M == 31) {
    return lane_xor<15>(lane_xor<16>(x));
  } else if constexpr (M > 32) {
    return lane_xor<M ^ 32>(lane_xor<32>(x));
  } else {
    // bitmask mode: lane' = ((lane & 0x1f) | 0) ^ M within each half of the wave
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, (M << 10) | 0x1F);
  }
}

template <int M> __device__ __forceinline__ uint64_t lane_xor64(uint64_t v) {
  const uint32_t lo = lane_xor<M>((uint32_t)v), hi = lane_xor<M>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t kmin(uint64_t a, uint64_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint64_t kmax(uint64_t a, uint64_t b) { return a < b ? b : a; }

// A run in a wave: k0 at position 2 * lane, k1 at 2 * lane + 1.
struct Run {
  uint64_t k0, k1;
};

// positions 2l and 2l + 1 (within the lane)
__device__ __forceinline__ void run_cas1(Run &r) {
  const bool sw = r.k1 < r.k0;
  const uint64_t lo = sw ? r.k1 : r.k0, hi = sw ? r.k0 : r.k1;
  r.k0 = lo;
  r.k1 = hi;
}

// One side of a compare-exchange: the lower position keeps the smaller key, the upper one
// the larger, so the partner's key y replaces k exactly when (y < k) == lower. (Equal keys
// are padding, where either is the same.) One 64-bit compare and two selects per key; the
// comparison with `lower` is an operation on lane masks.
__device__ __forceinline__ uint64_t keep(uint64_t k, uint64_t y, bool lower) {
  return (y < k) == lower ? y : k;
}

// Half-cleaner step of stride 2M: position p against p ^ 2M (lane ^ M, the same slot); the
// lower position keeps the smaller key.
template <int M> __device__ __forceinline__ void run_xor(Run &r, int lane) {
  const bool lower = (lane & M) == 0;
  r.k0 = keep(r.k0, lane_xor64<M>(r.k0), lower);
  r.k1 = keep(r.k1, lane_xor64<M>(r.k1), lower);
}

// First step of a merge of size 2M + 2: position p against p ^ (2M + 1), its mirror within
// the block (lane ^ M, the other slot); the lower position keeps the smaller key.
template <int M> __device__ __forceinline__ void run_mirror(Run &r, int lane) {
  const bool lower = (lane & ((M + 1) >> 1)) == 0;
  const uint64_t y0 = lane_xor64<M>(r.k1), y1 = lane_xor64<M>(r.k0);
  r.k0 = keep(r.k0, y0, lower);
  r.k1 = keep(r.k1, y1, lower);
}

// Sort a bitonic run ascending: half-cleaners of strides 64, 32, ..., 1.
__device__ __forceinline__ void run_clean(Run &r, int lane) {
  run_xor<32>(r, lane);
  run_xor<16>(r, lane);
  run_xor<8>(r, lane);
  run_xor<4>(r, lane);
  run_xor<2>(r, lane);
  run_xor<1>(r, lane);
  run_cas1(r);
}

// Sort an arbitrary run ascending (bitonic sort in the mirror form: every merge sorts
// ascending, so no element needs a direction).
__device__ __forceinline__ void run_sort(Run &r, int lane) {
  run_cas1(r);                                                      // blocks of 2
  run_mirror<1>(r, lane);  run_cas1(r);                             // 4
  run_mirror<3>(r, lane);  run_xor<1>(r, lane);  run_cas1(r);       // 8
  run_mirror<7>(r, lane);  run_xor<2>(r, lane);  run_xor<1>(r, lane);  run_cas1(r);  // 16
  run_mirror<15>(r, lane); run_xor<4>(r, lane);  run_xor<2>(r, lane);  run_xor<1>(r, lane);
  run_cas1(r);                                                      // 32
  run_mirror<31>(r, lane); run_xor<8>(r, lane);  run_xor<4>(r, lane);  run_xor<2>(r, lane);
  run_xor<1>(r, lane);     run_cas1(r);                             // 64
  run_mirror<63>(r, lane); run_xor<16>(r, lane); run_xor<8>(r, lane); run_xor<4>(r, lane);
  run_xor<2>(r, lane);     run_xor<1>(r, lane);  run_cas1(r);       // 128
}

// r <- the best 128 keys of r and the sorted run at src (128 keys), sorted. Lane l reads
// the pair at src[126 - 2l], src[127 - 2l]: the other run reversed.
__device__ __forceinline__ void run_merge_from(Run &r, const uint64_t *src, int lane) {
  const uint64_t b1 = src[126 - 2 * lane], b0 = src[127 - 2 * lane];
  r.k0 = kmin(r.k0, b0);
  r.k1 = kmin(r.k1, b1);
  run_clean(r, lane);
}

__device__ __forceinline__ void run_store(const Run &r, uint64_t *dst, int lane) {
  dst[2 * lane] = r.k0;
  dst[2 * lane + 1] = r.k1;
}

struct TopkRunArgs {
  const float *scores;      // [rows][n]
  int64_t n;
  const uint64_t *in_runs;  // merge passes: [rows][n_runs][RUN]
  int64_t n_runs;           // runs per row at the input of a merge pass
  uint64_t *out_runs;       // [rows][gridDim.x][RUN], or nullptr on the final pass
  int k;
  float *out_scores;        // final pass: [rows][k]
  int32_t *out_index;       // final pass: [rows][k]
};

// The 16 runs of the workgroup merge into wave 0's run (a tree through LDS); then wave 0
// writes either the row's top k or the workgroup's run.
__device__ __forceinline__ void run_tree_and_emit(Run r, const TopkRunArgs &a, int64_t row,
                                                  uint64_t (*lds)[RUN]) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = threadIdx.x >> 6;
  // At level `span`, wave w + span hands its run to wave w (w a multiple of 2 * span). The
  // slots written at one level are never those read at an earlier one, so one barrier per
  // level orders them.
#pragma unroll
  for (int span = 1; span < RUN_WAVES; span <<= 1) {
    if ((w & (2 * span - 1)) == span) run_store(r, lds[w], lane);
    __syncthreads();
    if ((w & (2 * span - 1)) == 0) run_merge_from(r, lds[w + span], lane);
  }
  if (w != 0) return;
  if (a.out_runs) {
    run_store(r, a.out_runs + (row * gridDim.x + blockIdx.x) * RUN, lane);
    return;
  }
  const uint64_t key[2] = {r.k0, r.k1};
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int e = 2 * lane + h;
    if (e < a.k) {
      const bool real = key[h] != ~0ull;
      const uint32_t idx = (uint32_t)key[h];
      a.out_scores[row * a.k + e] = real ? a.scores[row * a.n + idx] : -__builtin_inff();
      a.out_index[row * a.k + e] = real ? (int32_t)idx : -1;
    }
  }
}

// Pass 1: workgroup (chunk, row) takes scores [chunk * 2048, chunk * 2048 + 2048) of the row.
__global__ void __launch_bounds__(RUN_THREADS) topk_runs_kernel(TopkRunArgs a) {
  __shared__ uint64_t lds[RUN_WAVES][RUN];
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = threadIdx.x >> 6;
  const int64_t row = blockIdx.y;
  const int64_t i0 = (int64_t)blockIdx.x * RUN_CHUNK + w * RUN + 2 * lane;
  const float *src = a.scores + row * a.n;
  Run r;
  r.k0 = i0 < a.n ? ((uint64_t)topk_score_key(src[i0]) << 32) | (uint64_t)i0 : ~0ull;
  r.k1 = i0 + 1 < a.n ? ((uint64_t)topk_score_key(src[i0 + 1]) << 32) | (uint64_t)(i0 + 1) : ~0ull;
  run_sort(r, lane);
  run_tree_and_emit(r, a, row, lds);
}

// Later passes: workgroup (group, row) merges runs [group * 64, group * 64 + 64) of the row;
// wave w takes runs w, w + 16, w + 32, w + 48 in turn, then the tree.
__global__ void __launch_bounds__(RUN_THREADS) topk_merge_kernel(TopkRunArgs a) {
  __shared__ uint64_t lds[RUN_WAVES][RUN];
  const int lane = threadIdx.x & (WAVE - 1);
  const int w = threadIdx.x >> 6;
  const int64_t row = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * RUN_FANIN + w;
  const uint64_t *runs = a.in_runs + row * a.n_runs * RUN;
  // all of the wave's runs are loaded before the first merge (one memory latency, not four);
  // lane l holds run j's keys at positions 2l, 2l + 1 (the first) and, reversed, at
  // 127 - 2l, 126 - 2l (the others)
  constexpr int PER = RUN_FANIN / RUN_WAVES;
  uint64_t b0[PER], b1[PER];
#pragma unroll
  for (int j = 0; j < PER; j++) {
    const int64_t rj = r0 + j * RUN_WAVES;
    b0[j] = b1[j] = ~0ull;
    if (rj < a.n_runs) {
      const uint64_t *src = runs + rj * RUN;
      b0[j] = j == 0 ? src[2 * lane] : src[127 - 2 * lane];
      b1[j] = j == 0 ? src[2 * lane + 1] : src[126 - 2 * lane];
    }
  }
  Run r{b0[0], b1[0]};
#pragma unroll
  for (int j = 1; j < PER; j++) {
    if (r0 + j * RUN_WAVES < a.n_runs) {
      r.k0 = kmin(r.k0, b0[j]);
      r.k1 = kmin(r.k1, b1[j]);
      run_clean(r, lane);
    }
  }
  run_tree_and_emit(r, a, row, lds);
}

}  // namespace maxsim
