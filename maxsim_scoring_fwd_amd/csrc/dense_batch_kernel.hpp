// Several short queries against the same documents in one pass, one wave per document
// (TileMaxSim deep reading, section 2 item (1): tiling along queries as well as documents;
// Flash-MaxSim Figure 1: running max per query token, one fp32 score per pair).
//
//   out[q][b] = sum_i max_j <Q[q][i], d_j>   for every query q of the launch
//
// Design for gfx950:
//  * The queries of the launch (up to 16 blocks of 16 tokens, each query padded to whole
//    blocks) sit in LDS for the whole kernel, shared by the 8 waves of a workgroup, their
//    16-byte pieces XOR-swizzled by row as in the staged document tiles (conflict-free
//    128-bit reads; a padded row stride measured 4 conflict cycles per read).
//  * Each wave owns a document at a time and holds G of its 16-token tiles at once as
//    matrix-core A operands. Every query block read from LDS then feeds G tiles, so the
//    LDS traffic is one 1 KiB read per G MFMAs, and the loop has no workgroup barrier:
//    waves never wait for each other.
//  * The document stream is the dense kernel's: 1 KiB contiguous non-temporal loads of a
//    whole group of tiles, issued before the current group's products so they are in
//    flight meanwhile, transposed through a per-wave swizzled LDS tile. Tiles of a group
//    past the document's end load a dummy and take a copy of the last real tile (a
//    duplicate token cannot change a maximum); rows past the end clamp to the last token.
//  * The running max of each query token stays in one VGPR per query block; at the
//    document's end the row groups combine by cross-row swaps and each query's tokens are
//    summed over the 16 lanes of a row, in double, rounded once to fp32 (as the query-tiled
//    kernel does, so a single query scores the same with or without per-token outputs).
#pragma once

#include "dense_kernel.hpp"

namespace maxsim {

constexpr int DBATCH_THREADS = 512;
constexpr int DBATCH_WAVES = DBATCH_THREADS / WAVE;

// Wave-uniform state of one group of G tiles of one document.
struct TileGroup {
  int64_t doc;
  int nvalid;  // tiles inside the document; the rest copy the last of them
  bool valid, first, doc_end, empty;
};

template <int KSB, int NQB> constexpr size_t dense_batch_lds() {
  return (size_t)NQB * 16 * KSB * 64 + (size_t)DBATCH_WAVES * stage_tile_bytes<KSB>();
}

// DT: bf16 or fp16 storage; KSB: 64-byte chunks per row (the whole row, d * 2 bytes);
// G: document tiles per group; NQB: query blocks in LDS (n_q * ceil(q_len / 16) of them
// are real, the rest zero and never summed).
template <int DT, int KSB, int G, int NQB>
__global__ void __launch_bounds__(DBATCH_THREADS) dense_batch_kernel(DenseArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  static_assert(DT == DT_BF16 || DT == DT_FP16, "two-byte storage");
  constexpr int PPR = KSB * 4;  // 16-byte pieces per row
  static_assert((PPR & (PPR - 1)) == 0, "staged tiles need 2^k pieces");
  constexpr int64_t RB = KSB * 64;  // bytes per token row
  const int lane = threadIdx.x & (WAVE - 1);
  const int r16 = lane & 15, g = lane >> 4;
  const int wave_in_wg = threadIdx.x >> 6;
  const int64_t wave = uniform((int64_t)blockIdx.x * DBATCH_WAVES + wave_in_wg);
  const int64_t nwaves = (int64_t)gridDim.x * DBATCH_WAVES;
  char *tile = lds + NQB * 16 * RB + wave_in_wg * stage_tile_bytes<KSB>();
  const int q_len = a.q_len, n_q = a.n_q;

  // ---- queries into LDS: block qb, row r = token (qb % bpq) * 16 + r of query qb / bpq ----
  {
    constexpr int per_row = (int)(RB / 16);
    const int bpq = (q_len + 15) >> 4;  // query blocks per query
    for (int idx = threadIdx.x; idx < NQB * 16 * per_row; idx += DBATCH_THREADS) {
      const int row = idx / per_row, col = idx - row * per_row;
      const int qb = row >> 4, q = qb / bpq, tok = (qb - q * bpq) * 16 + (row & 15);
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (q < n_q && tok < q_len) v = load16(a.Q + ((int64_t)q * q_len + tok) * RB + col * 16);
      *reinterpret_cast<u32x4_t *>(lds + row * RB + (col ^ stage_swizzle<PPR>(row & 15)) * 16) = v;
    }
    __syncthreads();
  }

  // ---- producer: groups of G tiles of this wave's documents ----
  int64_t pb = wave, pend = a.n_docs, pstep = nwaves;
  if (a.offsets) {
    const int64_t t0 = uniform(a.offsets[0]);
    const int64_t ntok = uniform(a.offsets[a.n_docs]) - t0;
    const int64_t lo = t0 + ntok * wave / nwaves, hi = t0 + ntok * (wave + 1) / nwaves;
    pb = nearest_boundary(a.offsets, a.n_docs, lo, lane);
    pend = wave == nwaves - 1 ? a.n_docs : nearest_boundary(a.offsets, a.n_docs, hi, lane);
    if (wave == 0) pb = 0;
    pstep = 1;
  } else if (a.contiguous) {
    pb = a.n_docs * wave / nwaves;
    pend = a.n_docs * (wave + 1) / nwaves;
    pstep = 1;
  }
  int64_t pfirst = 0, plen = 0, ptile = 0;
  if (pb < pend) doc_extent(a, pb, pfirst, plen);

  u32x4_t buf[G][KSB];
  TileGroup nx;
  auto issue = [&]() {
    nx.valid = false;
    nx.nvalid = 0;
    const char *base = a.Q;  // in-bounds dummy source
    int64_t lastrow = 0;     // last valid row of the document, relative to base
    if (pb < pend) {
      nx.valid = true;
      nx.doc = pb;
      nx.first = ptile == 0;
      bool advance = true;
      if (plen == 0) {
        nx.empty = nx.doc_end = true;
      } else {
        nx.empty = false;
        const int64_t ntiles = (plen + 15) >> 4, left = ntiles - ptile;
        nx.nvalid = left < G ? (int)left : G;
        base = a.D + (pfirst + ptile * 16) * RB;
        lastrow = plen - 1 - ptile * 16;
        ptile += G;
        nx.doc_end = ptile >= ntiles;
        advance = nx.doc_end;
      }
      if (advance) {
        pb += pstep;
        ptile = 0;
        if (pb < pend) doc_extent(a, pb, pfirst, plen);
      }
    }
    // Tiles past the document (and every tile of an empty or exhausted group) read the
    // first query row: only wave-uniform values differ between the cases.
#pragma unroll
    for (int p = 0; p < G; p++) {
      const bool in = p < nx.nvalid;
      const char *bp = in ? base + (int64_t)p * 16 * RB : a.Q;
      const int64_t lr = lastrow - p * 16;
      const int last = in ? (lr < 15 ? (int)lr : 15) : 0;
#pragma unroll
      for (int c = 0; c < KSB; c++) {
        const int u = c * 64 + lane;
        const int row = u / PPR < last ? u / PPR : last;
        buf[p][c] = load16_nt(bp + (int64_t)row * RB + (u % PPR) * 16);
      }
    }
  };
  issue();

  float m[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; qb++) m[qb] = -__builtin_inff();

  for (;;) {
    const TileGroup cur = nx;
    if (!cur.valid) break;
    // transpose the group's tiles through LDS into A-operand layout (one token row per lane)
    u32x4_t aop[G][KSB];
#pragma unroll
    for (int p = 0; p < G; p++) {
#pragma unroll
      for (int c = 0; c < KSB; c++) {
        const int u = c * 64 + lane, row = u / PPR, piece = u % PPR;
        *reinterpret_cast<u32x4_t *>(tile + (row * PPR + (piece ^ stage_swizzle<PPR>(row))) * 16) =
            buf[p][c];
      }
#pragma unroll
      for (int c = 0; c < KSB; c++)
        aop[p][c] = *reinterpret_cast<const u32x4_t *>(
            tile + (r16 * PPR + ((4 * c + g) ^ stage_swizzle<PPR>(r16))) * 16);
    }
#pragma unroll
    for (int p = 1; p < G; p++)
      if (p >= cur.nvalid) {
#pragma unroll
        for (int c = 0; c < KSB; c++) aop[p][c] = aop[p - 1][c];
      }
    issue();  // the next group's loads run under this group's products

    if (cur.first) {
#pragma unroll
      for (int qb = 0; qb < NQB; qb++) m[qb] = -__builtin_inff();
    }
    if (!cur.empty) {
      // Software pipeline over the query blocks: block qb + 1's operands are read from LDS
      // before block qb's MFMAs, and block qb - 1's results are folded into its running max
      // while they run, so neither the LDS latency nor the matrix core's drain is waited for.
      u32x4_t bq[2][KSB];
      f32x4_t acc[2][G];
      auto read_b = [&](int qb, u32x4_t(&dst)[KSB]) {
#pragma unroll
        for (int c = 0; c < KSB; c++)
          dst[c] = *reinterpret_cast<const u32x4_t *>(
              lds + (qb * 16 + r16) * RB + ((4 * c + g) ^ stage_swizzle<PPR>(r16)) * 16);
      };
      auto fold = [&](int qb, const f32x4_t(&r)[G]) {
        float v = m[qb];
#pragma unroll
        for (int p = 0; p < G; p++) v = __builtin_fmaxf(v, max4(r[p]));
        m[qb] = v;
      };
      read_b(0, bq[0]);
#pragma unroll
      for (int qb = 0; qb < NQB; qb++) {
        const int cb = qb & 1;
        if (qb + 1 < NQB) read_b(qb + 1, bq[cb ^ 1]);
#pragma unroll
        for (int p = 0; p < G; p++) acc[cb][p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KSB; c++)
#pragma unroll
          for (int p = 0; p < G; p++) acc[cb][p] = ChunkMfma<DT>::run(aop[p][c], bq[cb][c], acc[cb][p]);
        if (qb > 0) fold(qb - 1, acc[cb ^ 1]);
        // order within the block: the next block's reads, G MFMAs, then the fold's vector
        // instructions one per MFMA (the earlier block's results are complete by then);
        // nothing moves across blocks
        if (qb + 1 < NQB) __builtin_amdgcn_sched_group_barrier(0x100, KSB, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, G, 0);
#pragma unroll
        for (int i = 0; i < (KSB - 1) * G; i++) {
          __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      fold(NQB - 1, acc[(NQB - 1) & 1]);
    }
    if (cur.doc_end) {
      // blocks in order: query q's tokens t0 .. t0 + 15 (wave-uniform counters). The maxima
      // are summed in double and rounded once, as in the query-tiled kernel.
      double s = 0.0;
      int q = 0, t0 = 0;
#pragma unroll
      for (int qb = 0; qb < NQB; qb++) {
        if (q >= n_q) break;
        const float v = max_row_groups(m[qb]);
        if (r16 < q_len - t0) s += (double)v;
        t0 += 16;
        if (t0 >= q_len) {
          s = sum_row16(s);
          if (lane == 0) a.out[(int64_t)q * a.n_docs + cur.doc] = cur.empty ? -__builtin_inff() : (float)s;
          s = 0.0;
          q++;
          t0 = 0;
        }
      }
    }
  }
}

}  // namespace maxsim
