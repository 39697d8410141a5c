// Product-quantisation MaxSim: per-query distance tables and fused lookup scoring.
//
// What it computes (TileMaxSim deep reading, section 2 item (3)):
//   T[i][m][k] = <segment m of q_i, C[m][k]>           (table build, once per query)
//   s_ij       = sum_m T[i][m][codes[j][m]]             (a token's similarity, by lookups)
//   out[b]     = sum_i max_{j in b} s_ij
// Codes are never expanded to vectors. The pages keep the table in on-chip
// shared memory; on gfx950 the fp32 tables of 32 query tokens (512 KiB) exceed
// the 160 KiB LDS, so the scorer stages one slice of 8 query tokens at a time.
//  * A workgroup of 16 waves owns one contiguous range of documents (token-balanced
//    for CSR corpora), cut into equal chunks of at most 512 documents (and, on
//    request, of at most a given number of tokens, small enough for their codes
//    to stay in L2). Each chunk is scored against every 8-query slice of the
//    tables in turn, the slice held in
//    LDS as TL[m][k][query] (the 8 queries of one (m, k) pair share 32 contiguous
//    bytes). Two threads score each token, four query tokens each: one 128-bit
//    LDS read per subspace fetches four table entries, so a wave instruction
//    serves 32 tokens.
//  * Each thread pair scores a contiguous run of the chunk's tokens, keeping the
//    running maxima of its four query tokens in registers; when the run crosses
//    into another document the maxima are folded into mx[doc][query] with LDS
//    float-max atomics. A max does not depend on order: scores are deterministic.
//  * After each slice a document's thread sums the slice's maxima in query order;
//    after the last slice it adds the slice sums in slice order and stores the
//    score.
//  * An empty document keeps -inf maxima and scores -inf.
#pragma once

#include "device_common.hpp"
#include "dense_kernel.hpp"
#include "host_common.hpp"

namespace maxsim {

constexpr int PQ_MAX_Q = 64;
constexpr int PQ_M = 16;
constexpr int PQ_K = 256;
constexpr int PQ_QS = 8;        // query tokens per LDS slice
constexpr int PQ_THREADS = 1024;
constexpr int PQ_CHUNK = 512;   // largest number of documents per chunk (LDS arrays)
constexpr int PQ_PAIRS = PQ_THREADS / 2;  // token lanes per workgroup (two threads each)

struct PqTableArgs {
  const char *Q;
  int q_len;
  int dtype;
  const float *C;
  int M, K, dsub;
  float *T;
};

struct PqScoreArgs {
  const float *T;
  int q_len;
  const uint8_t *codes;
  const int64_t *offsets;
  int64_t n_docs;
  int nd;
  float *out;
  int64_t chunk_tok = 0;  // largest number of tokens per chunk (0: documents only)
};

template <int DT> __device__ __forceinline__ float decode_elem(const char *Q, int64_t idx);
template <> __device__ __forceinline__ float decode_elem<DT_BF16>(const char *Q, int64_t idx) {
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(Q)[idx] << 16);
}
template <> __device__ __forceinline__ float decode_elem<DT_FP16>(const char *Q, int64_t idx) {
  return (float)reinterpret_cast<const _Float16 *>(Q)[idx];
}
template <> __device__ __forceinline__ float decode_elem<DT_FP32>(const char *Q, int64_t idx) {
  return reinterpret_cast<const float *>(Q)[idx];
}

// One thread per table entry; fp32 fused multiply-add over the dsub products.
template <int DT>
__global__ void __launch_bounds__(256) pq_tables_kernel(PqTableArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.q_len * a.M * a.K;
  if (idx >= total) return;
  const int64_t i = idx / ((int64_t)a.M * a.K);
  const int m = (int)((idx / a.K) % a.M);
  const int k = (int)(idx % a.K);
  const int64_t d = (int64_t)a.M * a.dsub;
  const float *c = a.C + ((int64_t)m * a.K + k) * a.dsub;
  float s = 0.f;
  for (int t = 0; t < a.dsub; t++) s = __builtin_fmaf(decode_elem<DT>(a.Q, i * d + (int64_t)m * a.dsub + t), c[t], s);
  a.T[idx] = s;
}

// A workgroup owns one contiguous range of documents: a token-balanced range for CSR
// documents (those starting in its share of the tokens, as in the dense kernel), an equal
// share of fixed-length documents otherwise. The range is cut into equal chunks of at most
// PQ_CHUNK documents and, when chunk_tok > 0, of at most chunk_tok tokens, so that a chunk's
// codes (16 bytes per token) can stay in L2 while the chunk is scored against every table
// slice. Chunks walk the slices up and down in turn (0..n-1, then n-1..0), so the
// slice at each chunk boundary is not staged again. Each document adds its slices'
// sums in slice order (kept in registers by the document's thread), each sum in query order.
constexpr int PQ_MAX_SLICES = PQ_MAX_Q / PQ_QS;
constexpr int PQ_STAGE = PQ_M * PQ_K / PQ_THREADS;  // (m, k) rows staged per thread
// LDS: 128 KiB of table slice + maxima (PQ_CHUNK x 8 queries) + offsets
static_assert(PQ_CHUNK < PQ_THREADS, "one thread per chunk offset");

__global__ void __launch_bounds__(PQ_THREADS) pq_score_kernel(PqScoreArgs a) {
  __shared__ __attribute__((aligned(16))) float tl[PQ_M * PQ_K * PQ_QS];  // 128 KiB: TL[m][k][query]
  __shared__ float mx[PQ_CHUNK * PQ_QS];        // maxima of the slice, per (document, query)
  __shared__ int32_t coff[PQ_CHUNK + 1];        // chunk-relative token offsets
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int pair = tid >> 1;                    // token lane: two threads per token
  const int h = tid & 1;                        // which 4 of the slice's 8 query tokens
  const int q_len = a.q_len;
  const int nslices = (q_len + PQ_QS - 1) / PQ_QS;
  const int64_t wg = blockIdx.x, nwg = gridDim.x;
  // this workgroup's documents [rb, re) (every wave computes the same range)
  int64_t rb, re;
  if (a.offsets) {
    const int64_t t0 = uniform(a.offsets[0]);
    const int64_t ntok = uniform(a.offsets[a.n_docs]) - t0;
    const int64_t lo = t0 + ntok * wg / nwg, hi = t0 + ntok * (wg + 1) / nwg;
    rb = wg == 0 ? 0 : uniform(wave_lower_bound(a.offsets, a.n_docs + 1, lo, lane));
    re = wg == nwg - 1 ? a.n_docs : uniform(wave_lower_bound(a.offsets, a.n_docs + 1, hi, lane));
  } else {
    rb = a.n_docs * wg / nwg;
    re = a.n_docs * (wg + 1) / nwg;
  }
  const int64_t nr = re > rb ? re - rb : 0;
  const int64_t rtok = nr == 0 ? 0
                       : a.offsets ? uniform(a.offsets[re]) - uniform(a.offsets[rb])
                                   : nr * (int64_t)a.nd;
  int64_t mine = (nr + PQ_CHUNK - 1) / PQ_CHUNK;  // chunks of the range
  if (a.chunk_tok > 0 && (rtok + a.chunk_tok - 1) / a.chunk_tok > mine)
    mine = (rtok + a.chunk_tok - 1) / a.chunk_tok;
  if (mine > nr) mine = nr;
  const int64_t cd = mine > 0 ? (nr + mine - 1) / mine : 1;  // documents per chunk (equal split)
  // first document and document count of this workgroup's chunk r
  auto chunk_docs = [&](int64_t r, int64_t &d0, int &ndc) {
    d0 = rb + r * cd;
    const int64_t left = re - d0;
    ndc = (int)(left < cd ? (left > 0 ? left : 0) : cd);
  };
  // the slice scored j-th in chunk r: up in even chunks, down in odd ones
  auto slice_at = [&](int64_t r, int j) { return (r & 1) ? nslices - 1 - j : j; };
  // TL[m][k][0..7] = T[q0 + 0..7][m][k]: this thread's PQ_STAGE (m, k) rows, loaded into
  // registers (neighbouring threads take neighbouring rows) and later written to LDS
  f32x4_t stage_lo[PQ_STAGE], stage_hi[PQ_STAGE];
  auto fetch = [&](int sl) {
    const int q0 = sl * PQ_QS;
#pragma unroll
    for (int i = 0; i < PQ_STAGE; i++) {
      const int mk = tid + i * PQ_THREADS;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        stage_lo[i][e] = q0 + e < q_len ? a.T[(int64_t)(q0 + e) * PQ_M * PQ_K + mk] : 0.f;
        stage_hi[i][e] = q0 + 4 + e < q_len ? a.T[(int64_t)(q0 + 4 + e) * PQ_M * PQ_K + mk] : 0.f;
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < PQ_STAGE; i++) {
      const int mk = tid + i * PQ_THREADS;
      *reinterpret_cast<f32x4_t *>(&tl[mk * PQ_QS]) = stage_lo[i];
      *reinterpret_cast<f32x4_t *>(&tl[mk * PQ_QS + 4]) = stage_hi[i];
    }
  };
  if (mine > 0) {
    fetch(slice_at(0, 0));
    store();
  }

  for (int64_t r = 0; r < mine; r++) {
    int64_t d0;
    int ndc;
    chunk_docs(r, d0, ndc);
    int64_t tok0 = 0;
    float psum[PQ_MAX_SLICES];  // thread tid < ndc: document d0 + tid's sum of each slice
#pragma unroll
    for (int s2 = 0; s2 < PQ_MAX_SLICES; s2++) psum[s2] = 0.f;
    for (int j = 0; j < nslices; j++) {
      const int sl = slice_at(r, j), q0 = sl * PQ_QS;
      const bool more = j + 1 < nslices || r + 1 < mine;
      const int next_sl = j + 1 < nslices ? slice_at(r, j + 1) : slice_at(r + 1, 0);
      const bool restage = more && next_sl != sl;
      __syncthreads();  // the previous slice is done with mx (and coff)
      if (j == 0) {
        if (a.offsets) {
          tok0 = a.offsets[d0];
          if (tid <= ndc) coff[tid] = (int32_t)(a.offsets[d0 + tid] - tok0);
        } else {
          tok0 = d0 * (int64_t)a.nd;
          if (tid <= ndc) coff[tid] = tid * a.nd;
        }
      }
      for (int idx = tid; idx < PQ_CHUNK * PQ_QS; idx += PQ_THREADS) mx[idx] = -__builtin_inff();
      __syncthreads();  // coff, mx and the slice's table are ready

      // this token lane's contiguous run of the chunk's tokens and the document holding
      // its first token (largest doc with coff[doc] <= t_begin, skipping empty ones)
      const int ntok = coff[ndc];
      const int span = (ntok + PQ_PAIRS - 1) / PQ_PAIRS;
      const int t_begin = pair * span < ntok ? pair * span : ntok;
      const int t_end = t_begin + span < ntok ? t_begin + span : ntok;
      if (t_begin < t_end) {
        int doc = 0;
        for (int lo = 0, hi = ndc; lo < hi;) {
          const int mid = (lo + hi + 1) >> 1;
          if (coff[mid] <= t_begin) lo = mid; else hi = mid - 1;
          doc = lo;
        }
        f32x4_t run = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
        u32x4_t cw = load16(reinterpret_cast<const char *>(a.codes) + (tok0 + t_begin) * PQ_M);
        for (int t = t_begin; t < t_end; t++) {
          const u32x4_t cur = cw;
          if (t + 1 < t_end)  // next token's codes in flight while this one is scored
            cw = load16(reinterpret_cast<const char *>(a.codes) + (tok0 + t + 1) * PQ_M);
          if (t >= coff[doc + 1]) {
            // this token starts a later document: fold the run into the finished one
#pragma unroll
            for (int e = 0; e < 4; e++)
              __hip_atomic_fetch_max(&mx[doc * PQ_QS + 4 * h + e], run[e], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
            do doc++; while (coff[doc + 1] <= t);
            run = f32x4_t{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
          }
          f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < PQ_M; m++) {
            const uint32_t k = (cur[m >> 2] >> ((m & 3) * 8)) & 0xffu;
            sc += *reinterpret_cast<const f32x4_t *>(&tl[(m * PQ_K + (int)k) * PQ_QS + 4 * h]);
          }
#pragma unroll
          for (int e = 0; e < 4; e++) run[e] = __builtin_fmaxf(run[e], sc[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; e++)
          __hip_atomic_fetch_max(&mx[doc * PQ_QS + 4 * h + e], run[e], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      // The next slice's table entries are loaded only now: issued before the token loop,
      // they would sit ahead of its code loads in the in-order load counter, and every
      // code wait would also wait for them.
      if (restage) fetch(next_sl);
      __syncthreads();  // the chunk's maxima for this slice are complete; tl is free
      if (tid < ndc) {
        float acc = 0.f;
        for (int q = 0; q < PQ_QS && q0 + q < q_len; q++) acc += mx[tid * PQ_QS + q];
#pragma unroll
        for (int s2 = 0; s2 < PQ_MAX_SLICES; s2++)
          if (s2 == sl) psum[s2] = acc;
      }
      if (restage) store();
    }
    if (tid < ndc) {
      float tot = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < PQ_MAX_SLICES; s2++)
        if (s2 < nslices) tot += psum[s2];
      a.out[d0 + tid] = tot;
    }
  }
}

inline int pq_tables_run(const PqTableArgs &a, const DeviceInfo &, hipStream_t st) {
  const int64_t total = (int64_t)a.q_len * a.M * a.K;
  const unsigned grid = (unsigned)((total + 255) / 256);
  switch (a.dtype) {
  case MAXSIM_BF16: hipLaunchKernelGGL(pq_tables_kernel<DT_BF16>, dim3(grid), dim3(256), 0, st, a); break;
  case MAXSIM_FP16: hipLaunchKernelGGL(pq_tables_kernel<DT_FP16>, dim3(grid), dim3(256), 0, st, a); break;
  case MAXSIM_FP32: hipLaunchKernelGGL(pq_tables_kernel<DT_FP32>, dim3(grid), dim3(256), 0, st, a); break;
  default: return MAXSIM_ERR_DTYPE;
  }
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

inline int pq_score_run(const PqScoreArgs &a, const DeviceInfo &di, hipStream_t st) {
  // One workgroup per CU (the table slice fills LDS), each with one contiguous range of
  // documents: one round, balanced by tokens for CSR corpora.
  const int bpc = blocks_per_cu((const void *)pq_score_kernel, PQ_THREADS, 0);
  const int64_t max_wg = (int64_t)bpc * di.cus;
  int64_t grid = a.n_docs < max_wg ? a.n_docs : max_wg;
  if (grid < 1) grid = 1;
  // Tokens per chunk (0: chunks limited by documents only, one chunk per workgroup at 100K
  // documents). A cap of 6144 tokens (96 KiB of codes per CU, 3 MiB for the 32 CUs of an
  // XCD, inside its 4 MiB L2) keeps each chunk's codes in L2 across the slices: fetched
  // bytes fall from 4.1x to 1.15x the code bytes, but every extra restaging of a 128 KiB
  // slice costs about 4.4 us and the CSR corpus took 0.409 ms against 0.342 ms (16384
  // tokens: 0.355 ms). The kernel is bound by its LDS lookups, not by HBM, so the default
  // keeps whole ranges; MAXSIM_PQ_CHUNK_TOK sets a cap (read at every call).
  const int chunk_tok = env_knob("MAXSIM_PQ_CHUNK_TOK", 0);
  PqScoreArgs ka = a;
  ka.chunk_tok = chunk_tok;
  log_launch("pq_score", (const void *)pq_score_kernel, grid, PQ_THREADS, 0, bpc);
  hipLaunchKernelGGL(pq_score_kernel, dim3((unsigned)grid), dim3(PQ_THREADS), 0, st, ka);
  return hipGetLastError() == hipSuccess ? MAXSIM_OK : MAXSIM_ERR_LAUNCH;
}

}  // namespace maxsim
