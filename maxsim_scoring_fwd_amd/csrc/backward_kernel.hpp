// Backward pass of MaxSim scoring: gradients of L = sum_b g_b * score_b.
//
// What it computes (Flash-MaxSim abstract and page: the training backward pass
// reuses the argmax locations of the forward; an inverse-grid CSR gives an
// atomic-free, destination-owned gradient reduction). With j*(b, i) the argmax
// of query token i in document b (tok_arg of the forward) the score is linear in
// Q and D away from ties, and
//   dD[b, j] = g_b * sum_{i : j*(b,i) = j} q_i     (a zero row where no query token chose j)
//   dQ[i]    = sum_b g_b * d_{b, j*(b,i)}
//
// Design for gfx950:
//  * dD (HBM-write-bound: every document token gets a row, most of them zero).
//    One wave owns one document at a time, so each output row has exactly one
//    writer. The wave builds the document's inverse grid in LDS: it counts the
//    query tokens that chose each document token, scans the counts into row
//    starts, and places the query indices into their rows in increasing order
//    (a stable placement: ranks among equal rows come from a scan of the 64
//    lanes' keys, not from atomics). Each lane then writes 16-byte chunks of the
//    rows; a chunk sums its row's query tokens in that fixed order and scales by
//    g_b once. Long documents are processed in segments of BWD_SEG tokens. CSR
//    documents are split into token-balanced contiguous ranges across waves.
//  * dQ (gathers q_len document rows per document). Each workgroup owns a block
//    of 4-element chunks of dQ and a contiguous range of documents, and adds
//    g_b times the chosen rows in document order into registers; the partial
//    sums go to a caller-provided workspace, one slice per range, and a second
//    kernel adds the slices in range order in double. No atomics anywhere, so
//    the results are the same on every run.
//  * An argmax outside [0, len_b) (the -1 of an empty document) contributes
//    nothing; no access leaves the document.
#pragma once

#include "dense_kernel.hpp"
#include "device_common.hpp"

namespace maxsim {

struct BwdArgs {
  const char *Q;
  int q_len;
  const char *D;
  const int64_t *offsets;  // CSR token offsets [n_docs + 1], or nullptr (fixed nd)
  int64_t n_docs;
  int nd;
  int d;
  const int32_t *tok_arg;  // [n_docs][q_len]
  const float *grad;       // [n_docs]
  char *dQ;                // [q_len][d] in the gradient type
  char *dD;                // [tokens][d] in the gradient type
  float *partial;          // dQ partial sums: [n_ranges][q_len * d]
  int n_ranges;
};

constexpr int BWD_THREADS = 256;
constexpr int BWD_WAVES = BWD_THREADS / WAVE;
constexpr int BWD_SEG = 1024;  // document tokens per inverse-grid segment
constexpr int BWD_MAX_Q = 1024;
constexpr int DQ_SLOTS = 4;                              // 4-element dQ chunks per thread
constexpr int DQ_CHUNKS_PER_WG = BWD_THREADS * DQ_SLOTS;  // 4096 dQ elements per workgroup
constexpr int DQ_DOCS = 4;                               // documents in flight per step

__device__ __forceinline__ void bwd_extent(const BwdArgs &a, int64_t b, int64_t &first,
                                           int64_t &len) {
  if (a.offsets) {
    const c_i64 *off = (const c_i64 *)a.offsets;
    first = uniform(off[b]);
    len = uniform(off[b + 1]) - first;
  } else {
    first = b * (int64_t)a.nd;
    len = a.nd;
  }
}

// Order the wave's LDS accesses before and after this point (a wave-level barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// E consecutive elements of storage type DT at p, as fp32 (p aligned to E elements).
template <int DT, int E>
__device__ __forceinline__ void load_f32(const char *p, float (&x)[E]) {
  if constexpr (DT == DT_FP32) {
#pragma unroll
    for (int h = 0; h < E / 4; h++) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t *>(p + 16 * h);
      x[4 * h] = v.x;
      x[4 * h + 1] = v.y;
      x[4 * h + 2] = v.z;
      x[4 * h + 3] = v.w;
    }
  } else {
    uint32_t w[E / 2];
    if constexpr (E == 8) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t *>(p);
      w[0] = v.x, w[1] = v.y, w[2] = v.z, w[3] = v.w;
    } else {
      static_assert(E == 4, "4 or 8 elements");
      const uint2 v = *reinterpret_cast<const uint2 *>(p);
      w[0] = v.x, w[1] = v.y;
    }
#pragma unroll
    for (int e = 0; e < E; e++) {
      const uint32_t h = (w[e / 2] >> (16 * (e & 1))) & 0xffffu;
      if constexpr (DT == DT_BF16)
        x[e] = __uint_as_float(h << 16);
      else
        x[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    }
  }
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Store 16 bytes of output type OT (E = 16 / element bytes values), non-temporal.
template <int OT, int E>
__device__ __forceinline__ void store_chunk(char *p, const float (&x)[E]) {
  u32x4_t v;
  if constexpr (OT == DT_FP32) {
    static_assert(E == 4, "fp32 chunk");
    v = u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                __float_as_uint(x[3])};
  } else {
    static_assert(E == 8, "16-bit chunk");
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; e++)
      h[e] = OT == DT_BF16 ? bf16_rne(x[e])
                           : (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[e]);
    v = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
}

// dD: one wave per document; DT the storage type of Q and D, OT the gradient type.
template <int DT, int OT>
__global__ void __launch_bounds__(BWD_THREADS) bwd_dd_kernel(BwdArgs a) {
  __shared__ int32_t cnt_lds[BWD_WAVES][BWD_SEG];      // counts, then placement cursors
  __shared__ int32_t off_lds[BWD_WAVES][BWD_SEG + 1];  // row starts of the inverse grid
  __shared__ int32_t idx_lds[BWD_WAVES][BWD_MAX_Q];    // query tokens grouped by row
  constexpr int IB = Elem<DT>::bytes;
  constexpr int OB = Elem<OT>::bytes;
  constexpr int E = 16 / OB;  // gradient elements per 16-byte output chunk
  const int lane = threadIdx.x & (WAVE - 1);
  const int wv = threadIdx.x >> 6;
  int32_t *cnt = cnt_lds[wv];
  int32_t *off = off_lds[wv];
  int32_t *idx = idx_lds[wv];
  const int64_t wave = uniform((int64_t)blockIdx.x * BWD_WAVES + wv);
  const int64_t nwaves = (int64_t)gridDim.x * BWD_WAVES;
  const int q_len = a.q_len;
  const int cpr = a.d / E;  // output chunks per row

  // documents of this wave: a token-balanced contiguous range (CSR) or a stride
  int64_t b = wave, bend = a.n_docs, bstep = nwaves;
  if (a.offsets) {
    const int64_t t0 = uniform(a.offsets[0]);
    const int64_t ntok = uniform(a.offsets[a.n_docs]) - t0;
    const int64_t lo = t0 + ntok * wave / nwaves, hi = t0 + ntok * (wave + 1) / nwaves;
    b = wave == 0 ? 0 : uniform(wave_lower_bound(a.offsets, a.n_docs + 1, lo, lane));
    bend = wave == nwaves - 1 ? a.n_docs
                              : uniform(wave_lower_bound(a.offsets, a.n_docs + 1, hi, lane));
    bstep = 1;
  }

  for (; b < bend; b += bstep) {
    int64_t first, len;
    bwd_extent(a, b, first, len);
    const float g = a.grad[b];
    const int32_t *arg = a.tok_arg + b * q_len;
    for (int64_t s0 = 0; s0 < len; s0 += BWD_SEG) {
      const int seg = (int)(len - s0 < BWD_SEG ? len - s0 : BWD_SEG);
      // 1. how many query tokens chose each row of the segment
      for (int j = lane; j < seg; j += WAVE) cnt[j] = 0;
      wave_lds_sync();
      for (int i = lane; i < q_len; i += WAVE) {
        const int64_t j = (int64_t)arg[i] - s0;
        if (j >= 0 && j < seg)
          __hip_atomic_fetch_add(&cnt[j], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
      }
      wave_lds_sync();
      // 2. row starts: exclusive scan of the counts; the counts become cursors (0)
      int carry = 0;
      for (int j0 = 0; j0 < seg; j0 += WAVE) {
        const int j = j0 + lane;
        const int c = j < seg ? cnt[j] : 0;
        int x = c;
#pragma unroll
        for (int sh = 1; sh < WAVE; sh <<= 1) {
          const int y = __shfl_up(x, sh);
          if (lane >= sh) x += y;
        }
        if (j < seg) {
          off[j] = carry + x - c;
          cnt[j] = 0;
        }
        carry += __shfl(x, WAVE - 1);
      }
      if (lane == 0) off[seg] = carry;
      wave_lds_sync();
      // 3. place the query tokens into their rows, in increasing query order
      for (int i0 = 0; i0 < q_len; i0 += WAVE) {
        const int i = i0 + lane;
        int key = -1;
        if (i < q_len) {
          const int64_t j = (int64_t)arg[i] - s0;
          if (j >= 0 && j < seg) key = (int)j;
        }
        const int nl = q_len - i0 < WAVE ? q_len - i0 : WAVE;
        int before = 0, after = 0;  // lanes of this chunk with the same row
        for (int l = 0; l < nl; l++) {
          const int kl = __builtin_amdgcn_readlane(key, l);
          if (kl == key) {
            before += l < lane;
            after += l > lane;
          }
        }
        if (key >= 0) idx[off[key] + cnt[key] + before] = i;
        wave_lds_sync();
        if (key >= 0 && after == 0) cnt[key] += before + 1;  // the row's last lane
        wave_lds_sync();
      }
      // 4. write the segment's rows; zero rows need no query reads
      char *dst = a.dD + (first + s0) * (int64_t)a.d * OB;
      const int nchunk = seg * cpr;
      for (int u = lane; u < nchunk; u += WAVE) {
        const int row = u / cpr, c = u - row * cpr;
        const int e0 = off[row], e1 = off[row + 1];
        float acc[E];
#pragma unroll
        for (int k = 0; k < E; k++) acc[k] = 0.f;
        for (int e = e0; e < e1; e++) {
          float x[E];
          load_f32<DT, E>(a.Q + ((int64_t)idx[e] * a.d + c * E) * IB, x);
#pragma unroll
          for (int k = 0; k < E; k++) acc[k] += x[k];
        }
#pragma unroll
        for (int k = 0; k < E; k++) acc[k] *= g;
        store_chunk<OT, E>(dst + (int64_t)u * 16, acc);
      }
      wave_lds_sync();  // the next segment reuses the wave's LDS
    }
  }
}

// dQ partial sums: grid (chunk blocks, document ranges).
template <int DT>
__global__ void __launch_bounds__(BWD_THREADS) bwd_dq_partial_kernel(BwdArgs a) {
  constexpr int IB = Elem<DT>::bytes;
  const int cpr = a.d / 4;
  const int total = a.q_len * cpr;  // 4-element chunks of dQ
  const int r = blockIdx.y;
  const int64_t b0 = a.n_docs * r / a.n_ranges, b1 = a.n_docs * (r + 1) / a.n_ranges;
  int qi[DQ_SLOTS], cc[DQ_SLOTS];
  bool ok[DQ_SLOTS];
  float acc[DQ_SLOTS][4];
#pragma unroll
  for (int s = 0; s < DQ_SLOTS; s++) {
    const int u = blockIdx.x * DQ_CHUNKS_PER_WG + s * BWD_THREADS + threadIdx.x;
    ok[s] = u < total;
    qi[s] = ok[s] ? u / cpr : 0;
    cc[s] = ok[s] ? u - qi[s] * cpr : 0;
#pragma unroll
    for (int k = 0; k < 4; k++) acc[s][k] = 0.f;
  }
  for (int64_t bb = b0; bb < b1; bb += DQ_DOCS) {
    int64_t first[DQ_DOCS], len[DQ_DOCS];
    float g[DQ_DOCS];
    int j[DQ_DOCS][DQ_SLOTS];
#pragma unroll
    for (int t = 0; t < DQ_DOCS; t++) {
      const int64_t b = bb + t;
      first[t] = 0;
      len[t] = 0;
      g[t] = 0.f;
      if (b < b1) {
        bwd_extent(a, b, first[t], len[t]);
        g[t] = a.grad[b];
      }
#pragma unroll
      for (int s = 0; s < DQ_SLOTS; s++)
        j[t][s] = (b < b1 && ok[s]) ? a.tok_arg[b * a.q_len + qi[s]] : -1;
    }
    // documents in order, so each chunk's sum has a fixed order
#pragma unroll
    for (int t = 0; t < DQ_DOCS; t++)
#pragma unroll
      for (int s = 0; s < DQ_SLOTS; s++) {
        if (j[t][s] >= 0 && j[t][s] < len[t]) {
          float x[4];
          load_f32<DT, 4>(a.D + ((first[t] + j[t][s]) * a.d + cc[s] * 4) * IB, x);
#pragma unroll
          for (int k = 0; k < 4; k++) acc[s][k] = __builtin_fmaf(g[t], x[k], acc[s][k]);
        }
      }
  }
  float *dst = a.partial + (int64_t)r * total * 4;
#pragma unroll
  for (int s = 0; s < DQ_SLOTS; s++) {
    const int u = blockIdx.x * DQ_CHUNKS_PER_WG + s * BWD_THREADS + threadIdx.x;
    if (ok[s])
      *reinterpret_cast<f32x4_t *>(dst + (int64_t)u * 4) =
          f32x4_t{acc[s][0], acc[s][1], acc[s][2], acc[s][3]};
  }
}

// dQ[e] = sum over ranges of the partial sums, in range order, in double; stored in the
// gradient type OT (rounded once, to nearest even).
template <int OT>
__global__ void __launch_bounds__(BWD_THREADS) bwd_dq_reduce_kernel(const float *partial,
                                                                    int n_ranges, int n_elem,
                                                                    char *dQ) {
  const int e = blockIdx.x * BWD_THREADS + threadIdx.x;
  if (e >= n_elem) return;
  double s = 0.0;
  for (int r = 0; r < n_ranges; r++) s += (double)partial[(int64_t)r * n_elem + e];
  const float f = (float)s;
  if constexpr (OT == DT_FP32)
    reinterpret_cast<float *>(dQ)[e] = f;
  else if constexpr (OT == DT_BF16)
    reinterpret_cast<uint16_t *>(dQ)[e] = (uint16_t)bf16_rne(f);
  else
    reinterpret_cast<_Float16 *>(dQ)[e] = (_Float16)f;
}

// Document ranges of the dQ partial sums: enough workgroups to fill the device
// (about 2048 with the chunk blocks), never more ranges than documents. A function
// of the sizes only, so the workspace and the summation order do not depend on
// the device.
inline int bwd_dq_ranges(int q_len, int d, int64_t n_docs) {
  const int chunks = q_len * (d / 4);
  const int blocks = (chunks + DQ_CHUNKS_PER_WG - 1) / DQ_CHUNKS_PER_WG;
  int64_t r = 2048 / blocks;
  if (r < 1) r = 1;
  if (r > n_docs) r = n_docs;
  return (int)r;
}

}  // namespace maxsim
