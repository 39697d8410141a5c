// Dense MaxSim kernel (bf16 / fp16 / fp32 storage, fixed or CSR documents).
//
// What it computes (TileMaxSim deep reading, section 1; Flash-MaxSim Figure 1):
//   out[b] = sum_i max_j <q_i, d_j>, one fp32 score per document, with the
//   similarity tile held in matrix-core accumulators and never stored.
//
// Design for gfx950 (differs from the pages' Triton/SRAM design where noted):
//  * One wave owns one document at a time and walks documents with a stride of
//    the number of waves in the grid (persistent grid sized to fill every CU).
//    Documents are independent units (Flash-MaxSim Figure 1: one program per
//    (query, document) pair); there is no cross-wave communication.
//  * All query tokens stay on chip for the whole kernel (TileMaxSim section 2
//    item (1): BQ = Nq, single pass), so every document byte is read from HBM
//    once. Up to 32 query tokens with d <= 256 live in VGPRs as ready-made MFMA
//    B operands; wider d keeps Q in LDS with a padded row stride (bank-conflict
//    free 128-bit reads).
//  * Document tiles are 16 tokens. Each lane loads 16-byte pieces of one token
//    row straight into the MFMA A-operand registers (no LDS round trip: each
//    element is used by exactly one lane, so staging through LDS would only add
//    traffic). A P-slot register ring keeps P tiles of loads in flight per wave;
//    every slot always issues its loads (a dummy in-bounds address once the
//    work is exhausted) so the compiler's vmcnt waits stay uniform.
//  * The embedding dimension is processed in blocks of KSB*64 bytes; partial
//    dot products accumulate in the fp32 accumulator across blocks before the
//    max (TileMaxSim section 2 item (2), dimension tiling).
//  * Rows past a document's end are clamped to its last token. A duplicated
//    token cannot change a maximum, so no masking arithmetic is needed and no
//    load ever leaves the document.
//  * The running max of each query token over the document's tokens stays in
//    one VGPR per 16-query block (Flash-MaxSim Figure 1: running max m, fp32
//    accumulator). At the document's end, two cross-lane max steps and a
//    16-lane sum give the score; one lane stores it.
#pragma once

#include "device_common.hpp"

namespace maxsim {

struct DenseArgs {
  const char *Q;
  int q_len;
  const char *D;
  const int64_t *offsets;  // CSR token offsets [n_docs + 1], or nullptr
  int64_t n_docs;
  int nd;                  // fixed layout: tokens per document slot
  const int32_t *doc_lens; // fixed layout: valid tokens per document, or nullptr
  int n_dblk;              // number of d blocks (1 when Q is in VGPRs)
  float *out;
};

constexpr int DENSE_THREADS = 256;

// Extent of document b: first token row and length (wave-uniform).
__device__ __forceinline__ void doc_extent(const DenseArgs &a, int64_t b, int64_t &first,
                                           int64_t &len) {
  if (a.offsets) {
    first = uniform(a.offsets[b]);
    len = uniform(a.offsets[b + 1]) - first;
  } else {
    first = b * (int64_t)a.nd;
    len = a.nd;
    if (a.doc_lens) {
      int64_t l = uniform(a.doc_lens[b]);
      len = l < 0 ? 0 : (l > a.nd ? a.nd : l);
    }
  }
}

// DT: storage type; KSB: 64-byte chunks per d block; QB: 16-query blocks;
// P: tiles in flight per wave; QLDS: query operand read from LDS.
template <int DT, int KSB, int QB, int P, bool QLDS>
__global__ void __launch_bounds__(DENSE_THREADS) dense_maxsim_kernel(DenseArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds_q[];
  const int lane = threadIdx.x & (WAVE - 1);
  const int r16 = lane & 15;  // tile row (document token) / query column
  const int g = lane >> 4;    // 16-byte piece within a 64-byte chunk
  const int64_t wave = uniform((int64_t)blockIdx.x * (DENSE_THREADS / WAVE) + (threadIdx.x >> 6));
  const int64_t nwaves = (int64_t)gridDim.x * (DENSE_THREADS / WAVE);
  const int n_dblk = QLDS ? a.n_dblk : 1;
  const int64_t RB = (int64_t)n_dblk * KSB * 64;  // bytes per token row
  const int q_len = a.q_len;

  // ---- query tokens, resident for the whole kernel ----
  u32x4_t qreg[QLDS ? 1 : QB][QLDS ? 1 : KSB];
  const int64_t QROWB = RB + 16;  // padded LDS row stride: 16 rows hit distinct banks
  if constexpr (!QLDS) {
#pragma unroll
    for (int qb = 0; qb < QB; qb++) {
      const int qi = qb * 16 + r16;
#pragma unroll
      for (int c = 0; c < KSB; c++) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (qi < q_len) v = load16(a.Q + qi * RB + c * 64 + g * 16);
        qreg[qb][c] = v;
      }
    }
  } else {
    const int64_t per_row = RB / 16;
    const int64_t total = (int64_t)QB * 16 * per_row;
    for (int64_t idx = threadIdx.x; idx < total; idx += DENSE_THREADS) {
      const int64_t row = idx / per_row, col = idx - row * per_row;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < q_len) v = load16(a.Q + row * RB + col * 16);
      *reinterpret_cast<u32x4_t *>(lds_q + row * QROWB + col * 16) = v;
    }
    __syncthreads();
  }

  // ---- producer: the (doc, tile, d-block) sequence of this wave ----
  int64_t pb = wave, pfirst = 0, plen = 0, ptile = 0;
  int pk = 0;
  auto next_doc = [&](int64_t b) {
    // Skip empty documents (score -inf: a max over no tokens).
    while (b < a.n_docs) {
      doc_extent(a, b, pfirst, plen);
      if (plen > 0) break;
      if (lane == 0) a.out[b] = -__builtin_inff();
      b += nwaves;
    }
    pb = b;
    ptile = 0;
    pk = 0;
  };
  next_doc(pb);

  u32x4_t buf[P][KSB];
  bool s_valid[P];
  int64_t s_doc[P];
  int s_dblk[P];
  bool s_first[P], s_last_blk[P], s_doc_end[P];

  auto issue = [&](u32x4_t(&dst)[KSB], bool &valid, int64_t &doc, int &dblk, bool &first_blk,
                   bool &last_blk, bool &doc_end) {
    valid = pb < a.n_docs;
    const char *base = a.Q;
    int64_t lane_off = g * 16;
    if (valid) {
      const int64_t t0 = ptile * 16;
      int64_t row = plen - 1 - t0;
      row = row < r16 ? row : r16;
      base = a.D + (pfirst + t0) * RB + (int64_t)pk * KSB * 64;
      lane_off = row * RB + g * 16;
      doc = pb;
      dblk = pk;
      first_blk = (pk == 0);
      last_blk = (pk == n_dblk - 1);
      const int64_t ntiles = (plen + 15) >> 4;
      doc_end = last_blk && (ptile == ntiles - 1);
      if (++pk == n_dblk) {
        pk = 0;
        if (++ptile == ntiles) next_doc(pb + nwaves);
      }
    }
#pragma unroll
    for (int c = 0; c < KSB; c++) dst[c] = load16(base + lane_off + c * 64);
  };

#pragma unroll
  for (int p = 0; p < P; p++)
    issue(buf[p], s_valid[p], s_doc[p], s_dblk[p], s_first[p], s_last_blk[p], s_doc_end[p]);

  f32x4_t acc[QB];
  float m[QB];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    m[qb] = -__builtin_inff();
    acc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (;;) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      if (!s_valid[p]) goto done;
      if (s_first[p]) {
#pragma unroll
        for (int qb = 0; qb < QB; qb++) acc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int c = 0; c < KSB; c++) {
#pragma unroll
        for (int qb = 0; qb < QB; qb++) {
          u32x4_t qv;
          if constexpr (QLDS)
            qv = *reinterpret_cast<const u32x4_t *>(
                lds_q + (qb * 16 + r16) * QROWB + ((int64_t)s_dblk[p] * KSB + c) * 64 + g * 16);
          else
            qv = qreg[qb][c];
          acc[qb] = ChunkMfma<DT>::run(buf[p][c], qv, acc[qb]);
        }
      }
      if (s_last_blk[p]) {
#pragma unroll
        for (int qb = 0; qb < QB; qb++) m[qb] = __builtin_fmaxf(m[qb], max4(acc[qb]));
      }
      if (s_doc_end[p]) {
        float s = 0.f;
#pragma unroll
        for (int qb = 0; qb < QB; qb++) {
          float v = m[qb];
          v = __builtin_fmaxf(v, __shfl_xor(v, 16));
          v = __builtin_fmaxf(v, __shfl_xor(v, 32));
          if (qb * 16 + r16 < q_len) s += v;
          m[qb] = -__builtin_inff();
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 8);
        if (lane == 0) a.out[s_doc[p]] = s;
      }
      issue(buf[p], s_valid[p], s_doc[p], s_dblk[p], s_first[p], s_last_blk[p], s_doc_end[p]);
    }
  }
done:
  return;
}

}  // namespace maxsim
