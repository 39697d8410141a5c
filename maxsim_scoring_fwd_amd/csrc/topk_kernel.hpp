// Top-k selection over the scores: the k best documents of each row of scores, ordered by
// score (descending), ties by document index (ascending).
//
// What it computes (the stage after scoring in late-interaction retrieval: TileMaxSim deep
// reading, sections 4 and 6 — the documents handed on are the best-scoring ones): for a row
// of n fp32 scores, the k entries that come first in the order (score descending, index
// ascending), in that order.
//
// Design for gfx950:
//  * Each candidate is one 64-bit key: the score mapped to an unsigned integer whose order
//    is the reverse of the float order (so a smaller key is a better score) in the high
//    half, the document index in the low half. One unsigned comparison then implements the
//    whole order, ties included, and the result is exact and the same on every run.
//  * A workgroup of 1024 threads sorts a chunk of 2048 keys in LDS with a bitonic network
//    and writes its first k. Chunks of a level run in parallel; each level divides the
//    candidates by 2048 / k, until one chunk holds them all. No atomics anywhere.
//  * Level 1 builds the keys straight from the score rows; later levels read the previous
//    level's keys from a caller-provided workspace. Rows (queries of a batch) are
//    independent: blockIdx.y is the row.
#pragma once

#include "device_common.hpp"

namespace maxsim {

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_CHUNK = 2 * TOPK_THREADS;  // keys sorted per workgroup
constexpr int TOPK_MAX_K = TOPK_THREADS;      // at most half a chunk survives a level

// fp32 score -> unsigned key, smaller for better scores (-inf last; NaN is not ordered).
__device__ __forceinline__ uint32_t topk_score_key(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t ascending = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~ascending;
}

__device__ __forceinline__ float topk_key_score(uint64_t key) {
  const uint32_t ascending = ~(uint32_t)(key >> 32);
  const uint32_t u = (ascending & 0x80000000u) ? (ascending & 0x7fffffffu) : ~ascending;
  return __uint_as_float(u);
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
      a.out_scores[row * keep + e] = real ? topk_key_score(v) : -__builtin_inff();
      a.out_index[row * keep + e] = real ? (int32_t)(uint32_t)v : -1;
    }
  }
}

}  // namespace maxsim
