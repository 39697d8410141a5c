// Dense MaxSim kernel (bf16 / fp16 / fp32 / int8 storage, fixed or CSR documents).
//
// What it computes (TileMaxSim deep reading, section 1; Flash-MaxSim Figure 1):
//   out[b] = sum_i max_j <q_i, d_j>, one fp32 score per document, with the
//   similarity tile held in matrix-core accumulators and never stored.
//
// Design for gfx950 (differs from the pages' Triton/SRAM design where noted):
//  * One wave owns one document at a time (Flash-MaxSim Figure 1: one program
//    per (query, document) pair); there is no cross-wave communication. The
//    grid is persistent, sized to fill every CU. Fixed-length documents are
//    walked with a stride of the number of waves, or, with at least four
//    documents per wave, as one contiguous range per wave. CSR documents of varying
//    length are split into contiguous, token-balanced document ranges: each
//    wave finds its range with a 64-way parallel search over the offsets, so
//    no wave is left with a long tail of work.
//  * All query tokens stay on chip for the whole kernel (TileMaxSim section 2
//    item (1): BQ = Nq, single pass), so every document byte is read from HBM
//    once. Up to 32 query tokens with d <= 256 live in VGPRs as ready-made MFMA
//    B operands; wider d keeps Q in LDS with a padded row stride (bank-conflict
//    free 128-bit reads).
//  * Document tiles are 16 tokens. A P-slot register ring keeps P tiles of
//    loads in flight per wave; every slot always issues its loads (a dummy
//    in-bounds address once the work is exhausted) so the compiler's vmcnt
//    waits stay uniform. Two ways to bring a tile to the matrix core:
//      - staged (default where the row is a power-of-two number of 16-byte
//        pieces): every load instruction reads 1 KiB of contiguous memory,
//        marked non-temporal since each byte is read once; the tile is then
//        transposed through a per-wave LDS buffer (XOR-swizzled, conflict-free)
//        into MFMA operand layout. Whole cache lines per instruction is what
//        lets streaming reads approach the HBM ceiling.
//      - direct: each lane loads its 16-byte pieces of one token row straight
//        into the MFMA A-operand registers (16 rows x 64 B per instruction).
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
//  * INT8 storage (Flash-MaxSim abstract: INT8 x INT8 with per-token scales): the tile
//    product is the exact int32 dot on the int8 matrix core (16x16x64, the same 64-byte
//    chunks and operand layout), and each similarity is fl32(fl32(dot) * fl32(q_scale[i] *
//    d_scale[j])) before the max, as in the query-tiled kernel. The scale of a lane's tile row
//    travels with the tile's loads in the ring, and the scale products of a tile come from
//    one 4-block 16x16x1 fp32 MFMA (exact: one product plus zero, rounded once).
//  * With ARG the kernel also writes each query token's maximum and the lowest
//    document index reaching it (the argmax the Flash-MaxSim backward pass
//    reuses): rows are folded in increasing order with a strict comparison, and
//    the row groups combine with ties going to the lower index, so a clamped
//    duplicate row past the end never wins over the token it copies.
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
  float *tok_max;          // ARG only: per-token maxima [n_docs][q_len]
  int32_t *tok_arg;        // ARG only: per-token argmax [n_docs][q_len]
  int contiguous = 0;      // fixed layout: wave w takes documents [B*w/W, B*(w+1)/W)
  const float *q_scale = nullptr;  // INT8: per query token
  const float *d_scale = nullptr;  // INT8: per document token (the rows of D)
  int n_q = 1;                     // several-query kernel: queries [n_q][q_len] in Q
};

constexpr int DENSE_THREADS = 256;
constexpr int DENSE_WAVES = DENSE_THREADS / WAVE;

// How document tiles reach the matrix core.
enum { LOAD_DIRECT = 0, LOAD_DIRECT_NT = 1, LOAD_STAGED = 2 };

// Bytes of the per-wave LDS transpose buffer (one 16-token tile of one d block).
template <int KSB> constexpr int stage_tile_bytes() { return 16 * KSB * 64; }

// LDS piece swizzle of a staged tile with PPR 16-byte pieces per row: rows
// 0..15 reading the same logical piece land on 16 distinct 16-byte bank groups.
template <int PPR> __device__ __forceinline__ int stage_swizzle(int row) {
  if constexpr (PPR >= 16)
    return row & 15;
  else
    return (row * PPR / 16) & (PPR - 1);
}

// Extent of document b: first token row and length (wave-uniform). The offsets
// and lengths are read through the constant address space so that they become
// scalar loads: a vector load here would make every wait on the tile loads in
// flight also wait for this one (vector loads complete in order).
typedef __attribute__((address_space(4))) const int64_t c_i64;
typedef __attribute__((address_space(4))) const int32_t c_i32;
__device__ __forceinline__ void doc_extent(const DenseArgs &a, int64_t b, int64_t &first,
                                           int64_t &len) {
  if (a.offsets) {
    const c_i64 *off = (const c_i64 *)a.offsets;
    first = uniform(off[b]);
    len = uniform(off[b + 1]) - first;
  } else {
    first = b * (int64_t)a.nd;
    len = a.nd;
    if (a.doc_lens) {
      int64_t l = uniform((int64_t)((const c_i32 *)a.doc_lens)[b]);
      len = l < 0 ? 0 : (l > a.nd ? a.nd : l);
    }
  }
}

// First index i in [0, n) with off[i] >= target, or n if none (off non-decreasing).
// Each round probes 64 evenly spaced entries with one vector load per lane and
// narrows the range 64-fold: about log64(n) dependent loads.
__device__ __forceinline__ int64_t wave_lower_bound(const int64_t *off, int64_t n, int64_t target,
                                                    int lane) {
  int64_t lo = 0, hi = n;  // answer in [lo, hi]
  while (lo < hi) {
    const int64_t step = (hi - lo + WAVE - 1) / WAVE;
    const int64_t idx = lo + (int64_t)lane * step;
    const bool less = idx < hi && off[idx] < target;
    const int cnt = __popcll(__ballot(less));  // probes below target form a prefix
    if (cnt == 0) return lo;
    const int64_t last_less = lo + (int64_t)(cnt - 1) * step;
    const int64_t next = last_less + step;
    lo = last_less + 1;
    hi = next < hi ? next : hi;
    lo = uniform(lo);
    hi = uniform(hi);
  }
  return lo;
}

// The document boundary nearest to token target: the first document starting at or after
// target, or the one before it when that starts closer below (wave-uniform). Neighbouring
// waves cut their ranges with the same rule, so every document belongs to one wave, and a
// long document straddling a cut adds at most half its length to either wave.
__device__ __forceinline__ int64_t nearest_boundary(const int64_t *off, int64_t n_docs,
                                                    int64_t target, int lane) {
  int64_t b = uniform(wave_lower_bound(off, n_docs + 1, target, lane));
  if (b > 0) {
    const c_i64 *o = (const c_i64 *)off;
    const int64_t below = uniform(o[b - 1]);
    const int64_t above = b <= n_docs ? uniform(o[b]) : below;
    if (b > n_docs || target - below < above - target) b--;
  }
  return b;
}

// Per-slot state of the load ring (wave-uniform). The flags are kept as separate
// booleans: packed into one integer they lead the compiler to wait for every
// load in flight before each tile, which serialises the ring.
struct Slot {
  int64_t doc;
  int dblk, tile;
  bool valid, first_blk, last_blk, doc_end, empty;
};

// DT: storage type; KSB: 64-byte chunks per d block; QB: 16-query blocks;
// P: tiles in flight per wave; QLDS: query operand read from LDS; LM: load mode;
// ARG: also write per-token maxima and argmax.
template <int DT, int KSB, int QB, int P, bool QLDS, int LM, bool ARG>
__global__ void __launch_bounds__(DENSE_THREADS) dense_maxsim_kernel(DenseArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr bool I8 = DT == DT_I8;
  static_assert(!I8 || !QLDS, "INT8 keeps the query in registers (one d block)");
  using AccT = typename AccType<I8>::type;
  constexpr int PPR = KSB * 4;  // 16-byte pieces per row of one d block
  static_assert(LM != LOAD_STAGED || (PPR & (PPR - 1)) == 0, "staged tiles need 2^k pieces");
  const int lane = threadIdx.x & (WAVE - 1);
  const int r16 = lane & 15;  // tile row (document token) / query column
  const int g = lane >> 4;    // 16-byte piece within a 64-byte chunk
  const int wave_in_wg = threadIdx.x >> 6;
  const int64_t wave = uniform((int64_t)blockIdx.x * DENSE_WAVES + wave_in_wg);
  const int64_t nwaves = (int64_t)gridDim.x * DENSE_WAVES;
  const int n_dblk = QLDS ? a.n_dblk : 1;
  const int64_t RB = (int64_t)n_dblk * KSB * 64;  // bytes per token row
  const int q_len = a.q_len;
  const int64_t QROWB = RB + 16;  // padded LDS row stride of Q: 16 rows hit distinct banks
  const int64_t q_lds_bytes = QLDS ? (int64_t)QB * 16 * QROWB : 0;
  char *tile = lds + q_lds_bytes + wave_in_wg * stage_tile_bytes<KSB>();

  // ---- query tokens, resident for the whole kernel ----
  u32x4_t qreg[QLDS ? 1 : QB][QLDS ? 1 : KSB];
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
  }
  // INT8: the B operand of the scale products (scale_products): the scale of column r16 of
  // query block g (0 for padding and for blocks past QB)
  float qsb = 0.f;
  if constexpr (I8) {
    static_assert(!I8 || QB <= 4, "one scale-product MFMA covers four query blocks");
    if (g < QB && g * 16 + r16 < q_len) qsb = a.q_scale[g * 16 + r16];
  }
  if constexpr (QLDS) {
    const int64_t per_row = RB / 16;
    const int64_t total = (int64_t)QB * 16 * per_row;
    for (int64_t idx = threadIdx.x; idx < total; idx += DENSE_THREADS) {
      const int64_t row = idx / per_row, col = idx - row * per_row;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row < q_len) v = load16(a.Q + row * RB + col * 16);
      *reinterpret_cast<u32x4_t *>(lds + row * QROWB + col * 16) = v;
    }
    __syncthreads();
  }

  // ---- producer: the (doc, tile, d-block) sequence of this wave ----
  // No loops and no stores here: an empty document becomes one slot flagged
  // SLOT_EMPTY whose score (-inf, a max over no tokens) the consumer writes.
  int64_t pb = wave, pend = a.n_docs, pstep = nwaves;
  if (a.offsets) {
    // contiguous token-balanced range: the documents starting in this wave's share
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
  int pk = 0;
  if (pb < pend) doc_extent(a, pb, pfirst, plen);

  u32x4_t buf[P][KSB];
  Slot slot[P];
  float dsc[I8 ? P : 1];  // INT8: the scale of row r16 of each slot's tile

  auto issue = [&](u32x4_t(&dst)[KSB], Slot &sl, float &ds) {
    sl.valid = false;
    const char *base = a.Q;  // in-bounds dummy source for empty or exhausted slots
    const float *sbase = a.q_scale;  // INT8: the tile's first row scale, or a dummy
    int last = 0;            // last valid row of the tile
    if (pb < pend) {
      sl.valid = true;
      sl.doc = pb;
      bool advance = true;
      if (plen == 0) {
        sl.dblk = sl.tile = 0;
        sl.first_blk = sl.last_blk = sl.doc_end = sl.empty = true;
      } else {
        const int64_t t0 = ptile * 16;
        const int64_t rem = plen - 1 - t0;
        last = rem < 15 ? (int)rem : 15;
        base = a.D + (pfirst + t0) * RB + (int64_t)pk * KSB * 64;
        if constexpr (I8) sbase = a.d_scale + pfirst + t0;
        const int64_t ntiles = (plen + 15) >> 4;
        sl.dblk = pk;
        sl.tile = (int)ptile;
        sl.empty = false;
        sl.first_blk = (pk == 0);
        sl.last_blk = (pk == n_dblk - 1);
        sl.doc_end = sl.last_blk && (ptile == ntiles - 1);
        advance = false;
        if (++pk == n_dblk) {
          pk = 0;
          if (++ptile == ntiles) advance = true;
        }
      }
      if (advance) {
        pb += pstep;
        ptile = 0;
        pk = 0;
        if (pb < pend) doc_extent(a, pb, pfirst, plen);
      }
    }
    // The same per-lane formula serves the dummy case (base = Q, last = 0: every lane
    // reads within the first query row), so only wave-uniform values differ.
    if constexpr (LM == LOAD_STAGED) {
#pragma unroll
      for (int c = 0; c < KSB; c++) {
        const int u = c * 64 + lane;  // linear 16-byte piece of the tile
        const int row = u / PPR < last ? u / PPR : last;
        dst[c] = load16_nt(base + (int64_t)row * RB + (u % PPR) * 16);
      }
    } else {
      const int row = r16 < last ? r16 : last;
      const int64_t off = (int64_t)row * RB + g * 16;
#pragma unroll
      for (int c = 0; c < KSB; c++)
        dst[c] = LM == LOAD_DIRECT_NT ? load16_nt(base + off + c * 64) : load16(base + off + c * 64);
    }
    if constexpr (I8) {
      // rows past the tile's last one take its scale, as their tokens duplicate it
      ds = sbase[r16 < last ? r16 : last];
    } else {
      (void)ds;
    }
  };

#pragma unroll
  for (int p = 0; p < P; p++) issue(buf[p], slot[p], dsc[I8 ? p : 0]);

  AccT acc[QB];
  float m[QB];
  int arg[ARG ? QB : 1];
#pragma unroll
  for (int qb = 0; qb < QB; qb++) {
    m[qb] = -__builtin_inff();
    if constexpr (ARG) arg[qb] = -1;
    acc[qb] = AccT{0, 0, 0, 0};
  }

  for (;;) {
#pragma unroll
    for (int p = 0; p < P; p++) {
      if (!slot[p].valid) goto done;
      u32x4_t aop[KSB];
      if constexpr (LM == LOAD_STAGED) {
        // transpose through LDS: linear pieces in, one token row per lane out
#pragma unroll
        for (int c = 0; c < KSB; c++) {
          const int u = c * 64 + lane, row = u / PPR, piece = u % PPR;
          *reinterpret_cast<u32x4_t *>(tile + (row * PPR + (piece ^ stage_swizzle<PPR>(row))) * 16) =
              buf[p][c];
        }
#pragma unroll
        for (int c = 0; c < KSB; c++)
          aop[c] = *reinterpret_cast<const u32x4_t *>(
              tile + (r16 * PPR + ((4 * c + g) ^ stage_swizzle<PPR>(r16))) * 16);
      } else {
#pragma unroll
        for (int c = 0; c < KSB; c++) aop[c] = buf[p][c];
      }
      if (slot[p].first_blk) {
#pragma unroll
        for (int qb = 0; qb < QB; qb++) acc[qb] = AccT{0, 0, 0, 0};
      }
#pragma unroll
      for (int c = 0; c < KSB; c++) {
#pragma unroll
        for (int qb = 0; qb < QB; qb++) {
          u32x4_t qv;
          if constexpr (QLDS)
            qv = *reinterpret_cast<const u32x4_t *>(
                lds + (qb * 16 + r16) * QROWB + ((int64_t)slot[p].dblk * KSB + c) * 64 + g * 16);
          else
            qv = qreg[qb][c];
          if constexpr (I8)
            acc[qb] = chunk_mfma_i8(aop[c], qv, acc[qb]);
          else
            acc[qb] = ChunkMfma<DT>::run(aop[c], qv, acc[qb]);
        }
      }
      if constexpr (I8) {
        if (slot[p].last_blk) {
          // fl32(fl32(dot) * fl32(q_scale * d_scale)) per similarity, then as below; the
          // scale products come from the matrix core, one MFMA per tile
          const int row0 = slot[p].tile * 16 + 4 * g;
          const f32x16_t sp = scale_products(dsc[I8 ? p : 0], qsb);
#pragma unroll
          for (int qb = 0; qb < QB; qb++) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; r++) v[r] = __fmul_rn((float)acc[qb][r], sp[4 * qb + r]);
            if constexpr (ARG) {
#pragma unroll
              for (int r = 0; r < 4; r++)
                if (v[r] > m[qb]) {
                  m[qb] = v[r];
                  arg[qb] = row0 + r;
                }
            } else {
              m[qb] = __builtin_fmaxf(__builtin_fmaxf(m[qb], v[0]), v[1]);
              m[qb] = __builtin_fmaxf(__builtin_fmaxf(m[qb], v[2]), v[3]);
            }
          }
        }
      } else if (slot[p].last_blk) {
        if constexpr (ARG) {
          // lane holds rows 4g .. 4g + 3 of the tile, in increasing order
          const int row0 = slot[p].tile * 16 + 4 * g;
#pragma unroll
          for (int qb = 0; qb < QB; qb++)
#pragma unroll
            for (int r = 0; r < 4; r++)
              if (acc[qb][r] > m[qb]) {
                m[qb] = acc[qb][r];
                arg[qb] = row0 + r;
              }
        } else {
#pragma unroll
          for (int qb = 0; qb < QB; qb++) m[qb] = __builtin_fmaxf(m[qb], max4(acc[qb]));
        }
      }
      if (slot[p].doc_end) {
        float s = 0.f;
#pragma unroll
        for (int qb = 0; qb < QB; qb++) {
          float v = m[qb];
          const int qi = qb * 16 + r16;
          if constexpr (ARG) {
            int j = arg[qb];
            argmax_row_groups(v, j);
            if (g == 0 && qi < q_len) {
              // an empty document's slot multiplied dummy data: report no token
              const int64_t o = slot[p].doc * q_len + qi;
              a.tok_max[o] = slot[p].empty ? -__builtin_inff() : v;
              a.tok_arg[o] = slot[p].empty ? -1 : j;
            }
            arg[qb] = -1;
          } else {
            v = max_row_groups(v);
          }
          if (qi < q_len) s += v;
          m[qb] = -__builtin_inff();
        }
        s = sum_row16(s);
        if (slot[p].empty) s = -__builtin_inff();
        if (lane == 0) a.out[slot[p].doc] = s;
      }
      issue(buf[p], slot[p], dsc[I8 ? p : 0]);
    }
  }
done:
  return;
}

}  // namespace maxsim
