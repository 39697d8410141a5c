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
//    g_b once; the query is read from LDS when it fits. Long documents are processed
//    in segments of at most BWD_SEG tokens. CSR documents are split into token-balanced
//    contiguous ranges across waves. For CSR queries of at most 64 tokens the grid is a
//    64-bit set of query tokens per row instead (one LDS OR per token, walked lowest bit
//    first: the same summation order).
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
  int doc_weight = 0;      // dD over CSR documents: per-document cost in tokens for balancing
  int short_sets = 1;      // dD, query in LDS, q_len <= 64: bit 0 chosen-token sets, bit 1
                           // no prefetch of the next document
};

constexpr int BWD_THREADS = 256;
constexpr int BWD_WAVES = BWD_THREADS / WAVE;
constexpr int BWD_SEG = 1024;  // longest inverse-grid segment (document tokens)
constexpr int BWD_Q_LDS_MAX = 48 * 1024;  // largest query copied to LDS (bytes)
constexpr int DQ_ELEMS_PER_WG = 4096;  // dQ elements per workgroup (16-byte chunks per thread)
// Documents in flight per step of a dQ thread. Measured at the ColBERT shape (dQ partial,
// CSR corpus / fixed Nd=128): 1, 2, 3, 4, 8 gave 147 / 137 / 134 / 179 / 175 us and
// 153 / 147 / 146 / 186 / 180 us, every instance at 8 waves per SIMD.
constexpr int DQ_DOCS = 3;
constexpr int DD_ROWS = 4;             // dD rows per lane with their gathers in flight
constexpr int DD_PRE = 2;              // chosen query rows per dD row gathered ahead

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

// fp32 -> 16-bit gradient bits, rounded to nearest even (gfx950 converts two values
// per instruction).
template <int OT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (OT == DT_BF16) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
  } else {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
  }
}

// Store 16 bytes of output type OT (E = 16 / element bytes values); NT: non-temporal.
template <int OT, int E, bool NT>
__device__ __forceinline__ void store_chunk(char *p, const float (&x)[E]) {
  u32x4_t v;
  if constexpr (OT == DT_FP32) {
    static_assert(E == 4, "fp32 chunk");
    v = u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                __float_as_uint(x[3])};
  } else {
    static_assert(E == 8, "16-bit chunk");
    v = u32x4_t{pack2<OT>(x[0], x[1]), pack2<OT>(x[2], x[3]), pack2<OT>(x[4], x[5]),
                pack2<OT>(x[6], x[7])};
  }
  if constexpr (NT)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
  else
    *reinterpret_cast<u32x4_t *>(p) = v;
}

// First index i in [0, n) with (off[i] - t0) + w * i >= target, or n if none: the lower
// bound of a target in the cumulative cost of documents [0, i) when a document costs w plus
// one per token (off non-decreasing). 64 probes per round, as wave_lower_bound.
__device__ __forceinline__ int64_t weighted_lower_bound(const int64_t *off, int64_t n, int64_t t0,
                                                        int64_t w, int64_t target, int lane) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t step = (hi - lo + WAVE - 1) / WAVE;
    const int64_t idx = lo + (int64_t)lane * step;
    const bool less = idx < hi && off[idx] - t0 + w * idx < target;
    const int cnt = __popcll(__ballot(less));
    if (cnt == 0) return lo;
    const int64_t last_less = lo + (int64_t)(cnt - 1) * step;
    const int64_t next = last_less + step;
    lo = uniform(last_less + 1);
    hi = uniform(next < hi ? next : hi);
  }
  return lo;
}

// Dynamic LDS of the dD kernel: the query as stored (QLDS) at offset 0, then per wave
// cnt[seg_cap], off[seg_cap + 1] and idx[q_len] (int32).
__host__ __device__ inline int bwd_dd_wave_ints(int seg_cap, int q_len) {
  return 2 * seg_cap + 1 + q_len;
}

// dD: one wave per document; DT the storage type of Q and D, OT the gradient type; QLDS:
// the query is copied to LDS once per workgroup (when it fits), else read through L2.
template <int DT, int OT, bool QLDS, bool NT>
__global__ void __launch_bounds__(BWD_THREADS) bwd_dd_kernel(BwdArgs a, int seg_cap,
                                                             int q_lds_bytes) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int IB = Elem<DT>::bytes;
  constexpr int OB = Elem<OT>::bytes;
  constexpr int E = 16 / OB;  // gradient elements per 16-byte output chunk
  const int lane = threadIdx.x & (WAVE - 1);
  const int wv = threadIdx.x >> 6;
  const int q_len = a.q_len, d = a.d;
  if constexpr (QLDS) {
    const int pieces = q_len * d * IB / 16;
    for (int p = threadIdx.x; p < pieces; p += BWD_THREADS)
      reinterpret_cast<u32x4_t *>(lds)[p] = load16(a.Q + (int64_t)p * 16);
    __syncthreads();
  }
  int32_t *cnt =
      reinterpret_cast<int32_t *>(lds + q_lds_bytes) + wv * bwd_dd_wave_ints(seg_cap, q_len);
  int32_t *off = cnt + seg_cap;
  int32_t *idx = off + seg_cap + 1;
  const int64_t wave = uniform((int64_t)blockIdx.x * BWD_WAVES + wv);
  const int64_t nwaves = (int64_t)gridDim.x * BWD_WAVES;
  const int cpr = d / E;  // output chunks per row
  // lanes -> (row, chunk): cpr divides 64 for d <= 256 (bf16 / fp16) and d <= 128 (fp32)
  const bool by_row = WAVE % cpr == 0;
  const int rpi = by_row ? WAVE / cpr : 0;
  const int my_c = by_row ? lane % cpr : 0, my_r = by_row ? lane / cpr : 0;

  auto q_chunk = [&](int i, int c, float (&x)[E]) {
    const int64_t o = ((int64_t)i * d + c * E) * IB;
    if constexpr (QLDS)
      load_f32<DT, E>(lds + o, x);
    else
      load_f32<DT, E>(a.Q + o, x);
  };

  // documents of this wave: a contiguous range (CSR) balanced on doc_weight per document
  // plus one per token, or a stride
  int64_t b = wave, bend = a.n_docs, bstep = nwaves;
  if (a.offsets) {
    const int64_t t0 = uniform(a.offsets[0]);
    const int64_t w = a.doc_weight;
    const int64_t total = uniform(a.offsets[a.n_docs]) - t0 + w * a.n_docs;
    const int64_t lo = total * wave / nwaves, hi = total * (wave + 1) / nwaves;
    b = wave == 0 ? 0 : uniform(weighted_lower_bound(a.offsets, a.n_docs + 1, t0, w, lo, lane));
    bend = wave == nwaves - 1 ? a.n_docs
                              : uniform(weighted_lower_bound(a.offsets, a.n_docs + 1, t0, w, hi, lane));
    bstep = 1;
  }

  if constexpr (QLDS) {
    if (q_len <= WAVE && (a.short_sets & 1)) {
      // Short queries, one token per lane: the query tokens that chose a row form a 64-bit
      // set (low word in cnt, high word in off), built with one LDS OR per token and walked
      // lowest bit first, so every row's sum keeps increasing query order (0 + first +
      // second ...), as in the general path, with no counting, scan or placement phase.
      // The next document's extent, weight and choices load while this one is written.
      uint32_t *lo = reinterpret_cast<uint32_t *>(cnt), *hi = reinterpret_cast<uint32_t *>(off);
      auto fetch = [&](int64_t bb, int64_t &f, int64_t &l, float &gg, int &k) {
        bwd_extent(a, bb, f, l);
        gg = a.grad[bb];
        k = lane < q_len ? a.tok_arg[bb * q_len + lane] : -1;
      };
      int64_t first = 0, len = 0;
      float g = 0.f;
      int key = -1;
      const bool pre = !(a.short_sets & 2);
      if (b < bend) fetch(b, first, len, g, key);
      for (; b < bend; b += bstep) {
        int64_t nfirst = 0, nlen = 0;
        float ng = 0.f;
        int nkey = -1;
        if (pre && b + bstep < bend) fetch(b + bstep, nfirst, nlen, ng, nkey);
        for (int64_t s0 = 0; s0 < len; s0 += seg_cap) {
          const int seg = (int)(len - s0 < seg_cap ? len - s0 : seg_cap);
          for (int j = lane; j < seg; j += WAVE) {
            lo[j] = 0u;
            hi[j] = 0u;
          }
          wave_lds_sync();
          const int64_t j = (int64_t)key - s0;
          if (j >= 0 && j < seg)
            __hip_atomic_fetch_or(lane < 32 ? &lo[j] : &hi[j], 1u << (lane & 31),
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
          wave_lds_sync();
          char *dst = a.dD + (first + s0) * (int64_t)d * OB;
          auto emit = [&](int row, int c) {
            uint64_t m = ((uint64_t)hi[row] << 32) | lo[row];
            float acc[E];
#pragma unroll
            for (int k = 0; k < E; k++) acc[k] = 0.f;
            while (m) {
              const int i = __builtin_ctzll(m);
              m &= m - 1;
              float x[E];
              q_chunk(i, c, x);
#pragma unroll
              for (int k = 0; k < E; k++) acc[k] += x[k];
            }
#pragma unroll
            for (int k = 0; k < E; k++) acc[k] *= g;
            store_chunk<OT, E, NT>(dst + ((int64_t)row * cpr + c) * 16, acc);
          };
          if (by_row) {
            for (int row = my_r; row < seg; row += rpi) emit(row, my_c);
          } else {
            for (int u = lane; u < seg * cpr; u += WAVE) emit(u / cpr, u % cpr);
          }
          wave_lds_sync();  // the next segment reuses the wave's LDS
        }
        if (!pre && b + bstep < bend) fetch(b + bstep, nfirst, nlen, ng, nkey);
        first = nfirst;
        len = nlen;
        g = ng;
        key = nkey;
      }
      return;
    }
  }

  for (; b < bend; b += bstep) {
    int64_t first, len;
    bwd_extent(a, b, first, len);
    const float g = a.grad[b];
    const int32_t *arg = a.tok_arg + b * q_len;
    for (int64_t s0 = 0; s0 < len; s0 += seg_cap) {
      const int seg = (int)(len - s0 < seg_cap ? len - s0 : seg_cap);
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
      // 4. write the segment's rows; a row nobody chose is zero and reads no query
      char *dst = a.dD + (first + s0) * (int64_t)d * OB;
      auto emit = [&](int row, int c) {
        const int e0 = off[row], e1 = off[row + 1];
        float acc[E];
#pragma unroll
        for (int k = 0; k < E; k++) acc[k] = 0.f;
        for (int e = e0; e < e1; e++) {
          float x[E];
          q_chunk(idx[e], c, x);
#pragma unroll
          for (int k = 0; k < E; k++) acc[k] += x[k];
        }
#pragma unroll
        for (int k = 0; k < E; k++) acc[k] *= g;
        store_chunk<OT, E, NT>(dst + ((int64_t)row * cpr + c) * 16, acc);
      };
      if (QLDS && by_row) {
        for (int row = my_r; row < seg; row += rpi) emit(row, my_c);
      } else if (by_row) {
        // The query is gathered through L2 (too large for LDS), DD_ROWS rows per lane at a
        // time, software-pipelined: the first DD_PRE chosen query rows of each row of the
        // next batch (query row 0 where there are fewer) are gathered before this batch's
        // stores are issued. gfx9 retires vector memory operations in order, so a gather
        // issued after a store is waited for together with that store; issued before, it only
        // waits for the stores of the batch before. Rows past the segment's end are clamped to
        // its last row, so every batch issues the same number of gathers and stores (the
        // compiler's waits then count exactly); a clamped lane writes that row's chunk again
        // with the same bytes. Rows chosen more often gather the rest in order afterwards, and
        // every row sums 0 + first + second ..., so results are unchanged. (With the query in
        // LDS the batching's registers cost more occupancy than they save: CSR dD measured 2%
        // slower.)
        if (my_r < seg) {
          const int step = rpi * DD_ROWS;
          auto rows_of = [&](int row0, int (&rw)[DD_ROWS], int (&f0)[DD_ROWS], int (&f1)[DD_ROWS]) {
#pragma unroll
            for (int u = 0; u < DD_ROWS; u++) {
              const int row = row0 + u * rpi < seg ? row0 + u * rpi : seg - 1;
              rw[u] = row;
              f0[u] = off[row];
              f1[u] = off[row + 1];
            }
          };
          auto gather_first = [&](const int (&f0)[DD_ROWS], const int (&f1)[DD_ROWS],
                                  float (&xx)[DD_ROWS][DD_PRE][E]) {
#pragma unroll
            for (int u = 0; u < DD_ROWS; u++)
#pragma unroll
              for (int p = 0; p < DD_PRE; p++)  // query row 0: a safe dummy
                q_chunk(f0[u] + p < f1[u] ? idx[f0[u] + p] : 0, my_c, xx[u][p]);
          };
          int rw[DD_ROWS], f0[DD_ROWS], f1[DD_ROWS];
          float xf[DD_ROWS][DD_PRE][E];
          rows_of(my_r, rw, f0, f1);
          gather_first(f0, f1, xf);
          // Wait for the first batch here (vmcnt(0); expcnt and lgkmcnt unconstrained), so
          // the loop is entered with no gather pending, as at its back-edge: otherwise the
          // compiler's wait for a batch's gathers, merged over both ways into the loop, would
          // also wait for the previous batch's stores.
          __builtin_amdgcn_s_waitcnt(0x0F70);
          for (int row0 = my_r;; row0 += step) {
            const bool more = row0 + step < seg;
            int nw[DD_ROWS], n0[DD_ROWS], n1[DD_ROWS];
            float xn[DD_ROWS][DD_PRE][E];
            rows_of(more ? row0 + step : row0, nw, n0, n1);  // the last batch gathers itself again
            gather_first(n0, n1, xn);
            float acc[DD_ROWS][E];
#pragma unroll
            for (int u = 0; u < DD_ROWS; u++) {
#pragma unroll
              for (int k = 0; k < E; k++) acc[u][k] = 0.f;
#pragma unroll
              for (int p = 0; p < DD_PRE; p++)
#pragma unroll
                for (int k = 0; k < E; k++) acc[u][k] += f0[u] + p < f1[u] ? xf[u][p][k] : 0.f;
            }
            // rows chosen by more than DD_PRE query tokens: the rest in order (rare)
#pragma unroll
            for (int u = 0; u < DD_ROWS; u++)
              for (int e = f0[u] + DD_PRE; e < f1[u]; e++) {
                float x[E];
                q_chunk(idx[e], my_c, x);
#pragma unroll
                for (int k = 0; k < E; k++) acc[u][k] += x[k];
              }
#pragma unroll
            for (int u = 0; u < DD_ROWS; u++) {
#pragma unroll
              for (int k = 0; k < E; k++) acc[u][k] *= g;
              store_chunk<OT, E, NT>(dst + ((int64_t)rw[u] * cpr + my_c) * 16, acc[u]);
            }
            if (!more) break;
#pragma unroll
            for (int u = 0; u < DD_ROWS; u++) {
              rw[u] = nw[u];
              f0[u] = n0[u];
              f1[u] = n1[u];
#pragma unroll
              for (int p = 0; p < DD_PRE; p++)
#pragma unroll
                for (int k = 0; k < E; k++) xf[u][p][k] = xn[u][p][k];
            }
          }
        }
      } else {
        for (int u = lane; u < seg * cpr; u += WAVE) emit(u / cpr, u % cpr);
      }
      wave_lds_sync();  // the next segment reuses the wave's LDS
    }
  }
}

// dQ partial sums: grid (element blocks, document ranges). Each thread owns SLOTS chunks
// of 16 bytes of the stored type (E elements each) of dQ and adds g_b times the chosen
// rows' chunks for the documents of its range, in document order.
template <int DT, int DOCS = DQ_DOCS>
__global__ void __launch_bounds__(BWD_THREADS) bwd_dq_partial_kernel(BwdArgs a) {
  constexpr int IB = Elem<DT>::bytes;
  constexpr int E = 16 / IB;
  constexpr int SLOTS = DQ_ELEMS_PER_WG / (BWD_THREADS * E);
  const int cpr = a.d / E;
  const int total = a.q_len * cpr;  // chunks of dQ
  const int r = blockIdx.y;
  const int64_t b0 = a.n_docs * r / a.n_ranges, b1 = a.n_docs * (r + 1) / a.n_ranges;
  int qi[SLOTS], cc[SLOTS];
  bool ok[SLOTS];
  float acc[SLOTS][E];
#pragma unroll
  for (int s = 0; s < SLOTS; s++) {
    const int u = blockIdx.x * (BWD_THREADS * SLOTS) + s * BWD_THREADS + threadIdx.x;
    ok[s] = u < total;
    qi[s] = ok[s] ? u / cpr : 0;
    cc[s] = ok[s] ? u - qi[s] * cpr : 0;
#pragma unroll
    for (int k = 0; k < E; k++) acc[s][k] = 0.f;
  }
  for (int64_t bb = b0; bb < b1; bb += DOCS) {
    int64_t first[DOCS], len[DOCS];
    float g[DOCS];
    int j[DOCS][SLOTS];
#pragma unroll
    for (int t = 0; t < DOCS; t++) {
      const int64_t b = bb + t;
      first[t] = 0;
      len[t] = 0;
      g[t] = 0.f;
      if (b < b1) {
        bwd_extent(a, b, first[t], len[t]);
        g[t] = a.grad[b];
      }
#pragma unroll
      for (int s = 0; s < SLOTS; s++)
        j[t][s] = (b < b1 && ok[s]) ? a.tok_arg[b * a.q_len + qi[s]] : -1;
    }
    // documents in order, so each chunk's sum has a fixed order
#pragma unroll
    for (int t = 0; t < DOCS; t++)
#pragma unroll
      for (int s = 0; s < SLOTS; s++) {
        if (j[t][s] >= 0 && j[t][s] < len[t]) {
          float x[E];
          load_f32<DT, E>(a.D + ((first[t] + j[t][s]) * a.d + cc[s] * E) * IB, x);
#pragma unroll
          for (int k = 0; k < E; k++) acc[s][k] = __builtin_fmaf(g[t], x[k], acc[s][k]);
        }
      }
  }
  float *dst = a.partial + (int64_t)r * total * E;
#pragma unroll
  for (int s = 0; s < SLOTS; s++) {
    const int u = blockIdx.x * (BWD_THREADS * SLOTS) + s * BWD_THREADS + threadIdx.x;
    if (ok[s]) {
#pragma unroll
      for (int h = 0; h < E / 4; h++)
        *reinterpret_cast<f32x4_t *>(dst + (int64_t)u * E + 4 * h) =
            f32x4_t{acc[s][4 * h], acc[s][4 * h + 1], acc[s][4 * h + 2], acc[s][4 * h + 3]};
    }
  }
}

// dQ[e] = sum over ranges of the partial sums in double; stored in the gradient type OT
// (rounded once, to nearest even). A workgroup takes RED_ELEMS consecutive elements; its
// RED_GROUPS thread groups each add every RED_GROUPS-th range in increasing order, and the
// group sums are added in group order: a fixed order, whatever the timing.
constexpr int RED_ELEMS = 16;
constexpr int RED_GROUPS = BWD_THREADS / RED_ELEMS;
template <int OT>
__global__ void __launch_bounds__(BWD_THREADS) bwd_dq_reduce_kernel(const float *partial,
                                                                    int n_ranges, int n_elem,
                                                                    char *dQ) {
  __shared__ double red[RED_GROUPS][RED_ELEMS];
  const int el = threadIdx.x % RED_ELEMS, grp = threadIdx.x / RED_ELEMS;
  const int e = blockIdx.x * RED_ELEMS + el;
  double s = 0.0;
  if (e < n_elem) {
#pragma unroll 8
    for (int r = grp; r < n_ranges; r += RED_GROUPS) s += (double)partial[(int64_t)r * n_elem + e];
  }
  red[grp][el] = s;
  __syncthreads();
  if (grp != 0 || e >= n_elem) return;
  double tot = 0.0;
  for (int k = 0; k < RED_GROUPS; k++) tot += red[k][el];
  const float f = (float)tot;
  if constexpr (OT == DT_FP32)
    reinterpret_cast<float *>(dQ)[e] = f;
  else
    reinterpret_cast<uint16_t *>(dQ)[e] = (uint16_t)(pack2<OT>(f, 0.f) & 0xffffu);
}

// Document ranges of the dQ partial sums: enough workgroups to fill the device
// (about 2048 with the element blocks), never more ranges than documents. A function
// of the sizes only, so the workspace and the summation order do not depend on
// the device.
inline int bwd_dq_ranges(int q_len, int d, int64_t n_docs) {
  const int blocks = (q_len * d + DQ_ELEMS_PER_WG - 1) / DQ_ELEMS_PER_WG;
  int64_t r = 2048 / blocks;
  if (r < 1) r = 1;
  if (r > n_docs) r = n_docs;
  return (int)r;
}

}  // namespace maxsim
