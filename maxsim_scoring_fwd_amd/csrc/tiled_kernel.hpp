// Query-tiled MaxSim kernel: long queries (ColPali shape) and INT8 x INT8.
//
// What it computes: out[b] = sum_i max_j s(q_i, d_j) with
//   - s = <q_i, d_j> for bf16 / fp16 / fp32 storage (TileMaxSim deep reading,
//     section 1), or
//   - s = fl32( fl32(dot_ij) * fl32(q_scale[i] * d_scale[j]) ) for int8 storage,
//     dot_ij the exact int32 dot product (Flash-MaxSim abstract: INT8xINT8
//     scoring; the per-token scales are applied as a product before the max).
//     The scale products fl32(q_scale[i] * d_scale[j]) of a 16-token tile are an
//     outer product with one term per entry: the matrix core computes them
//     (v_mfma_f32_16x16x1_4b_f32, four 16x16 blocks with K = 1, each entry one
//     product plus zero, rounded once to nearest even, so bit-identical to a
//     rounded multiply) in the layout of the int32 accumulators, and the vector
//     unit keeps one convert, one rounded multiply and half a three-way max per
//     similarity.
//
// Flash-MaxSim's forward pass (Figure 1, Algorithm 2) loops over query tiles
// inside one program per (query, document) pair; on gfx950 the query tiles run
// concurrently instead: the NW waves of a workgroup (8, or 4 for queries of up to 384 tokens)
// each hold one slice of the query tokens as resident MFMA B operands (QBW blocks
// of 16 tokens), and one copy of every document block sits in LDS for all of them.
//  * Documents are walked by workgroup (grid stride). A block is 32 KiB of
//    document tokens: each wave loads 32 / NW KiB of it with 1 KiB contiguous,
//    non-temporal loads, writes it to a double-buffered XOR-swizzled LDS tile
//    and, after one barrier, every wave reads the block's 16-token tiles as
//    A operands. The next block's loads are in flight while the current one is
//    multiplied, and each document is read from HBM once for all query slices.
//  * Rows past the document's end are clamped to its last token (a duplicate
//    cannot change a maximum); whole tiles past the end are skipped.
//  * Per tile and query block, the 16x16 accumulator is reduced into a running
//    max held in one VGPR per lane (plus the argmax when per-token maxima and
//    argmax are asked for: the lowest row reaching the maximum).
//  * At the document's end each wave sums its maxima per query; the partial sums
//    meet in LDS and each query adds them in wave order. These sums over up to
//    1024 query tokens are taken in double and rounded once to fp32, so a score of
//    a few hundred keeps its fp32 precision.
//  * Several queries can share one pass over the documents (each padded to whole
//    16-token blocks): every document byte then serves n_q queries, and each query
//    gets its own score per document.
#pragma once

#include "device_common.hpp"
#include "dense_kernel.hpp"

namespace maxsim {

constexpr int TILED_WAVES = 8;  // default waves per workgroup (query slices)
constexpr int TILED_BLOCK_BYTES = 32 * 1024;


struct TiledArgs {
  const char *Q;
  int q_len;
  const char *D;
  const int64_t *offsets;   // CSR, or nullptr for fixed documents of nd tokens
  int64_t n_docs;
  int nd;
  const int32_t *doc_lens;  // fixed layout only, nullable
  const float *q_scale;     // int8 only
  const float *d_scale;     // int8 only, per document token
  float *out;
  float *tok_max;           // ARG only: per-token maxima [n_docs][q_len]
  int32_t *tok_arg;         // ARG only: per-token argmax [n_docs][q_len]
  int n_q = 1;              // queries of q_len tokens each, Q [n_q][q_len][d], out [n_q][n_docs]
};

__device__ __forceinline__ void tiled_extent(const TiledArgs &a, int64_t b, int64_t &first,
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

// DT: storage; KSB: 64-byte chunks per token row (d = KSB * 64 / element bytes);
// QBW: 16-query blocks per wave (queries per workgroup = 8 * 16 * QBW);
// ARG: also produce the per-token maxima and argmax (single query); NW: waves per
// workgroup; BATCH: several queries (TiledArgs::n_q), else exactly one.
template <int DT, int KSB, int QBW, bool ARG, int NW = TILED_WAVES, bool BATCH = false>
__global__ void __launch_bounds__(NW * WAVE) tiled_maxsim_kernel(TiledArgs a) {
  static_assert(!(ARG && BATCH), "per-token outputs come with a single query");
  constexpr int TILED_THREADS = NW * WAVE;
  constexpr int RB = KSB * 64;                         // bytes per token row
  constexpr int PPR = KSB * 4;                         // 16-byte pieces per row
  constexpr int BLK_ROWS = TILED_BLOCK_BYTES / RB;     // tokens per block
  constexpr int BLK_TILES = BLK_ROWS / 16;
  constexpr int LOADS = TILED_BLOCK_BYTES / (TILED_THREADS * 16);  // per lane per block
  constexpr bool I8 = DT == DT_I8;
  static_assert((PPR & (PPR - 1)) == 0, "swizzle needs a power-of-two row");
  static_assert(!I8 || TILED_THREADS >= BLK_ROWS, "one thread per row stages the INT8 scales");
  __shared__ __attribute__((aligned(16))) char blk_lds[2][TILED_BLOCK_BYTES];
  __shared__ double part_lds[NW * QBW];  // per (wave, query) segment: its sum of maxima
  __shared__ __attribute__((aligned(16))) float dscale_lds[2][I8 ? BLK_ROWS : 4];

  const int lane = threadIdx.x & (WAVE - 1);
  const int r16 = lane & 15, g = lane >> 4;
  const int w = uniform((int)(threadIdx.x >> 6));
  const int q_len = a.q_len;
  const int q_pad = (q_len + 15) & ~15;  // each query padded to whole 16-token blocks
  const int q_base = w * QBW * 16;

  // ---- this wave's query slice, resident as B operands ----
  // Token t of the workgroup's numbering is token t % q_pad of query t / q_pad; padding
  // tokens are zero vectors and are left out of the sums.
  u32x4_t qreg[QBW][KSB];
  // INT8 scale products on the matrix core (SP) where the registers allow: the products of
  // a tile take 16 VGPRs per four query blocks. The widest slices (QBW * KSB > 16, d = 256
  // and 512 with long queries) form them on the vector unit instead (no spills).
  constexpr bool SP = I8 && QBW * KSB <= 16;
  // SP: lane l's B operand of the scale products of query blocks 4s .. 4s + 3: the scale of
  // column l % 16 of block 4s + l / 16 (0 for padding). Otherwise qs: the scale of the
  // lane's column of each block.
  constexpr int NS = SP ? (QBW + 3) / 4 : 1;
  float qsb[NS];
  float qs[SP ? 1 : QBW];
  // Row of Q [n_q * q_len] held by the lane's column of query block qb, or -1 (padding).
  // A 16-token block lies within one padded query, so the query index is wave-uniform.
  // (A single query: the row is the token index itself.)
  auto q_row = [&](int qb) -> int {
    if constexpr (!BATCH) {
      const int qi = q_base + qb * 16 + r16;
      return qi < q_len ? qi : -1;
    }
    const int tb = uniform(q_base + qb * 16);
    const int qq = tb / q_pad, pos = tb - qq * q_pad + r16;
    return qq < a.n_q && pos < q_len ? qq * q_len + pos : -1;
  };
  static_assert(!I8 || !BATCH, "INT8 scores one query per call");
#pragma unroll
  for (int s = 0; s < NS; s++) {
    qsb[s] = 0.f;
    if constexpr (SP) {
      const int qi = q_base + (4 * s + g) * 16 + r16;
      if (4 * s + g < QBW && qi < q_len) qsb[s] = a.q_scale[qi];
    }
  }
#pragma unroll
  for (int qb = 0; qb < QBW; qb++) {
    const int row = q_row(qb);
    if constexpr (I8 && !SP) qs[qb] = row >= 0 ? a.q_scale[row] : 0.f;
#pragma unroll
    for (int c = 0; c < KSB; c++) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (row >= 0) v = load16(a.Q + (int64_t)row * RB + c * 64 + g * 16);
      qreg[qb][c] = v;
    }
  }

  // The query of each of the wave's blocks (wave-uniform) and whether the lane's column of
  // it holds a token (bit qb), taken once: the work at every document's end then divides
  // nothing by q_pad (runtime divisions are long scalar sequences).
  int blk_q[QBW];
  uint32_t real_bits = 0;
#pragma unroll
  for (int qb = 0; qb < QBW; qb++) {
    blk_q[qb] = BATCH ? uniform((q_base + qb * 16) / q_pad) : 0;
    if (q_row(qb) >= 0) real_bits |= 1u << qb;
  }

  // ---- block sequence of this workgroup: (doc, block) in order ----
  // A cursor names block blk of document b (its first token and length); b >= n_docs ends
  // the sequence.
  struct Cursor {
    int64_t b, first, len;
    int blk;
  };
  auto first_block = [&](int64_t b) {
    Cursor c{b, 0, 0, 0};
    if (b < a.n_docs) tiled_extent(a, b, c.first, c.len);
    return c;
  };
  auto next_block = [&](const Cursor &c) {
    const int64_t nblk = c.len == 0 ? 1 : (c.len + BLK_ROWS - 1) / BLK_ROWS;
    if (c.blk == nblk - 1) return first_block(c.b + gridDim.x);
    Cursor n = c;
    n.blk++;
    return n;
  };

  // The next block's pieces are loaded into registers while the current one is multiplied.
  u32x4_t pre[LOADS];
  float pre_scale = 0.f;
  // Issue the loads of block c into pre (and its INT8 scales into pre_scale); a dummy
  // in-bounds read of the query when there is nothing to load.
  auto load_block = [&](const Cursor &c) {
    const bool real = c.b < a.n_docs && c.len > 0;
    const char *base = a.Q;
    int last = 0;
    if (real) {
      const int64_t r0 = (int64_t)c.blk * BLK_ROWS;
      const int64_t rem = c.len - 1 - r0;
      last = rem < BLK_ROWS - 1 ? (int)rem : BLK_ROWS - 1;
      base = a.D + (c.first + r0) * RB;
    }
#pragma unroll
    for (int k = 0; k < LOADS; k++) {
      const int u = (k * NW + w) * 64 + lane;  // linear 16-byte piece of the block
      const int row = u / PPR < last ? u / PPR : last;
      pre[k] = load16_nt(base + (int64_t)row * RB + (u % PPR) * 16);
    }
    if constexpr (I8) {
      if (threadIdx.x < BLK_ROWS) {
        const int row = (int)threadIdx.x < last ? (int)threadIdx.x : last;
        pre_scale = real ? a.d_scale[c.first + (int64_t)c.blk * BLK_ROWS + row] : 0.f;
      }
    }
  };
  Cursor cur = first_block(blockIdx.x);  // the next block to load
  Cursor meta = cur;                     // the block held by pre
  load_block(cur);
  cur = next_block(cur);

  float m[QBW];
  int arg[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; qb++) {
    m[qb] = -__builtin_inff();
    arg[qb] = -1;
  }
  int buf = 0;
  // A two-stage pipeline over the tiles (see the tile loop) where the registers allow a
  // second accumulator set (the query slice takes QBW * KSB * 4 VGPRs, each accumulator set
  // QBW * 4): INT8, whose vector work per tile outweighs its MFMAs, and the 4-wave dense
  // instances (short queries, two workgroups per CU), whose slices are small.
  constexpr bool PIPE = QBW * KSB <= 16 && (I8 || NW == 4);
  // The 8-wave dense instances of the several-query pass pipeline by halves of the query
  // slice (no extra registers). Measured: 32 ColBERT queries +6%; the single long query
  // (ColPali shape, the same loop) -3%, so it keeps the plain loop, except with the argmax,
  // whose fold is heavier (a compare and two selects per similarity): +1-2% there.
  constexpr bool HALF = (BATCH || ARG) && !PIPE && !I8 && NW >= TILED_WAVES && QBW % 2 == 0;
  using AccT = typename AccType<I8>::type;

  // Several queries whose blocks never straddle two waves ("local"): each segment of a wave
  // is a whole query, and the wave stores that query's score itself (no LDS, no barrier).
  // Its document-end work then leaves the critical path: the scores are stored after the
  // next block's barrier, so the wait for that block's loads does not include the stores,
  // and the waves of the second half of the workgroup, which share their SIMDs with the
  // first half, also take their reductions there, while the other wave of the SIMD
  // multiplies (with 4 waves, two independent workgroups share each SIMD instead). The
  // sums and their order are those of the immediate form.
  const bool local = BATCH && QBW % (q_pad / 16) == 0;
  const bool defer = local && NW >= TILED_WAVES && w >= NW / 2;
  bool pend_epi = false, pend_empty = false;  // deferred reductions of document pend_epi_b
  int64_t pend_epi_b = 0, pend_b = 0;
  float pend_v = 0.f;  // lane k: the k-th pending score of the wave (document pend_b)
  int pend_q = -1;     //   and its query, or -1
  auto local_epilogue = [&](int64_t b, bool empty) {
    double s = 0.0;
    int seg_q = blk_q[0], k = 0;
    auto flush = [&]() {
      s = sum_row16(s);
      if (lane == k) {
        pend_v = empty ? -__builtin_inff() : (float)s;
        pend_q = seg_q;
      }
      k++;
      s = 0.0;
    };
#pragma unroll
    for (int qb = 0; qb < QBW; qb++) {
      const float v = max_row_groups(m[qb]);
      const int qq = blk_q[qb];
      if (qq != seg_q) {
        flush();
        seg_q = qq;
      }
      if (((real_bits >> qb) & 1u) && !empty) s += (double)v;
      m[qb] = -__builtin_inff();
    }
    flush();
    pend_b = b;
  };
  // With 4 or 8 query blocks per wave and queries of 1, 2 or 4 blocks, the document end
  // treats every block at once. The row groups exchange their partial maxima so that row
  // group g ends with the whole maximum of block g (and of block g + 4): v_permlane16_swap
  // of blocks 2k and 2k + 1 leaves the pair's maximum of block 2k in the even row groups and
  // of block 2k + 1 in the odd ones, and v_permlane32_swap does the same across the halves
  // of the wave. Each 16-lane row then sums its block over the query tokens in double, and
  // the rows of one query's blocks add their sums. One exchange and one row sum serve four
  // blocks, where the form above reduces every block over the row groups and then every
  // query over the lanes. The same terms are summed in another order (in double), so the two
  // forms agree to the rounding of the fp32 scores.
  constexpr bool EPI4 = BATCH && (QBW == 4 || QBW == 8);
  const int bpq = q_pad / 16;  // blocks per query
  const bool epi4 = EPI4 && local && (bpq == 1 || bpq == 2 || bpq == 4);
  const int bpq_log = bpq == 4 ? 2 : (bpq == 2 ? 1 : 0);
  auto local_epilogue4 = [&](int64_t b, bool empty) {
    if constexpr (EPI4) {
      constexpr int NP = QBW / 2, NX = QBW / 4;
      float pm[NP];  // even row groups: block 2k, odd: block 2k + 1, over the pair
#pragma unroll
      for (int k = 0; k < NP; k++) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(m[2 * k]),
                                                        __float_as_uint(m[2 * k + 1]), false, false);
        pm[k] = __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
      }
#pragma unroll
      for (int k = 0; k < NX; k++) {
        // row group g: the maximum of column r16 of block 4k + g over all four row groups
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm[2 * k]),
                                                        __float_as_uint(pm[2 * k + 1]), false, false);
        const float x = __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
        const int blk_g = 4 * k + g;
        double s = ((real_bits >> blk_g) & 1u) ? (double)x : 0.0;
        s = sum_row16(s);
        if (bpq >= 2) s = pair_sum_f64<16>(s);
        if (bpq == 4) s = pair_sum_f64<32>(s);
        // lane k of the first row group of each query records its score
        if (r16 == k && (g & (bpq - 1)) == 0) {
          pend_v = empty ? -__builtin_inff() : (float)s;
          pend_q = blk_q[0] + (blk_g >> bpq_log);
        }
      }
#pragma unroll
      for (int qb = 0; qb < QBW; qb++) m[qb] = -__builtin_inff();
      pend_b = b;
    }
  };
  auto doc_epilogue = [&](int64_t b, bool empty) {
    if (epi4)
      local_epilogue4(b, empty);
    else
      local_epilogue(b, empty);
  };
  auto local_store = [&]() {
    if (pend_q >= 0 && pend_q < a.n_q) a.out[(int64_t)pend_q * a.n_docs + pend_b] = pend_v;
    pend_q = -1;
  };

  // byte offset of this lane's A-operand piece c within a staged 16-row tile
  int a_off[KSB];
#pragma unroll
  for (int c = 0; c < KSB; c++)
    a_off[c] = (r16 * PPR + ((4 * c + g) ^ stage_swizzle<PPR>(r16))) * 16;

  while (meta.b < a.n_docs) {
    // this block: stage the prefetched pieces in LDS
    char *tile = blk_lds[buf];
#pragma unroll
    for (int k = 0; k < LOADS; k++) {
      const int u = (k * NW + w) * 64 + lane, row = u / PPR, piece = u % PPR;
      *reinterpret_cast<u32x4_t *>(tile + (row * PPR + (piece ^ stage_swizzle<PPR>(row))) * 16) =
          pre[k];
    }
    if constexpr (I8) {
      if (threadIdx.x < BLK_ROWS) dscale_lds[buf][threadIdx.x] = pre_scale;
    }
    const int64_t b = meta.b, len = meta.len;
    const int blk = meta.blk;
    const bool empty = len == 0;
    const int64_t nblk = empty ? 1 : (len + BLK_ROWS - 1) / BLK_ROWS;
    const bool doc_end = (blk == nblk - 1);
    // prefetch the next block (of this or the next document)
    meta = cur;
    load_block(cur);
    cur = next_block(cur);
    __syncthreads();
    if constexpr (BATCH) {
      if (local) {
        if (pend_epi) {
          doc_epilogue(pend_epi_b, pend_empty);
          pend_epi = false;
        }
        local_store();
      }
    }

    // multiply the block's valid tiles against this wave's query slice
    if (!empty) {
      const int64_t rows_left = len - (int64_t)blk * BLK_ROWS;
      const int ntiles = rows_left >= BLK_ROWS ? BLK_TILES : (int)((rows_left + 15) >> 4);
      // A operand of chunk c of tile t: row t * 16 + r16, pieces 4c .. 4c + 3
      // (row t * 16 + r16 has the swizzle of row r16, so the lane's offset within a tile,
      // a_off[c], is fixed and tile t adds t * 16 rows)
      auto read_a = [&](int t, int c) -> u32x4_t {
        return *reinterpret_cast<const u32x4_t *>(tile + t * (16 * PPR * 16) + a_off[c]);
      };
      // all query blocks' accumulators are live: consecutive MFMAs are independent
      auto mfma_tile = [&](AccT(&acc)[QBW], const u32x4_t(&aop)[KSB]) {
#pragma unroll
        for (int qb = 0; qb < QBW; qb++) acc[qb] = AccT{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < KSB; c++)
#pragma unroll
          for (int qb = 0; qb < QBW; qb++) {
            if constexpr (I8)
              acc[qb] = chunk_mfma_i8(aop[c], qreg[qb][c], acc[qb]);
            else
              acc[qb] = ChunkMfma<DT>::run(aop[c], qreg[qb][c], acc[qb]);
          }
      };
      // tile t's similarities (INT8: the int32 dots scaled per row) folded into the running
      // max; with the argmax, ties keep the lowest row (the lane holds rows 4g .. 4g + 3 of
      // the tile in increasing order, and rows past the end duplicate the last token, so
      // only a strictly larger value replaces the maximum and their index is never taken)
      // INT8: the scale products of tile t (see scale_products), from the matrix core
      f32x16_t sp[NS];
      auto scale_tile = [&](int t) {
        if constexpr (SP) {
          const float ds = dscale_lds[buf][t * 16 + r16];
#pragma unroll
          for (int s = 0; s < NS; s++) sp[s] = scale_products(ds, qsb[s]);
        }
      };
      auto fold = [&](int t, const AccT(&acc)[QBW]) {
        const int row0 = t * 16 + 4 * g;
        f32x4_t ds;
        if constexpr (I8 && !SP) ds = *reinterpret_cast<const f32x4_t *>(&dscale_lds[buf][row0]);
#pragma unroll
        for (int qb = 0; qb < QBW; qb++) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; r++) {
            if constexpr (SP)
              v[r] = __fmul_rn((float)acc[qb][r], sp[qb / 4][4 * (qb % 4) + r]);
            else if constexpr (I8)
              v[r] = __fmul_rn((float)acc[qb][r], __fmul_rn(qs[qb], ds[r]));
            else
              v[r] = acc[qb][r];
          }
          if constexpr (ARG) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
              if (v[r] > m[qb]) {
                m[qb] = v[r];
                arg[qb] = blk * BLK_ROWS + row0 + r;
              }
            }
          } else if constexpr (I8) {
            m[qb] = __builtin_fmaxf(__builtin_fmaxf(m[qb], v[0]), v[1]);
            m[qb] = __builtin_fmaxf(__builtin_fmaxf(m[qb], v[2]), v[3]);
          } else {
            m[qb] = __builtin_fmaxf(m[qb], max4(acc[qb]));
          }
        }
      };
      if constexpr (PIPE) {
        // Two accumulator sets: the MFMAs of tile t + 1 are issued before tile t's vector
        // work (which then needs no result still in the matrix core), and the A operands
        // of tile t + 2 are read before it too.
        AccT accA[QBW], accB[QBW];
        u32x4_t an[KSB];  // A operands of the next tile to multiply
        // (a read past the last valid tile re-reads it: the steady state has no branches)
        auto read_next = [&](int t) {
          const int tt = t < ntiles ? t : ntiles - 1;
#pragma unroll
          for (int c = 0; c < KSB; c++) an[c] = read_a(tt, c);
        };
        // one MFMA, then a share of the vector work, in turn: a wave keeps the matrix core
        // and the vector unit busy at once
        auto interleave = [&]() {
          // vector instructions per query block: INT8 ~14 (per row a convert, two products,
          // and half a three-way max), the argmax ~12 (a compare and two selects per row),
          // a plain max ~4
          // INT8 ~10 per query block with the scale products on the matrix core (per row a
          // convert and a product, and half a three-way max), 14 without
          constexpr int VQB = SP ? 10 : I8 ? 14 : (ARG ? 12 : 4);
          constexpr int VPM = (VQB + KSB - 1) / KSB;
          __builtin_amdgcn_sched_group_barrier(0x100, KSB, 0);  // the A reads first
#pragma unroll
          for (int i = 0; i < QBW * KSB; i++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
          }
        };
        read_next(0);
        mfma_tile(accA, an);
        read_next(1);
        int t = 0;
        for (; t + 2 < ntiles; t += 2) {  // fold tiles t, t + 1; multiply t + 1, t + 2
          scale_tile(t);
          mfma_tile(accB, an);
          read_next(t + 2);
          fold(t, accA);
          interleave();
          scale_tile(t + 1);
          mfma_tile(accA, an);
          read_next(t + 3);
          fold(t + 1, accB);
          interleave();
        }
        if (t + 1 < ntiles) {  // two tiles left: t in accA, t + 1 in an
          scale_tile(t);
          mfma_tile(accB, an);
          fold(t, accA);
          scale_tile(t + 1);
          fold(t + 1, accB);
        } else {
          scale_tile(t);
          fold(t, accA);
        }
      } else if constexpr (HALF) {
        // No registers for a second accumulator set: the query blocks of a tile are taken in
        // two halves, and each half's MFMAs are interleaved with the folding of the other
        // half, whose results were issued half a tile earlier. The next tile's A operands
        // are read as soon as the current tile's last MFMA has taken them.
        constexpr int H = QBW / 2;
        AccT accA[H], accB[H];  // query blocks 0 .. H-1 and H .. QBW-1
        u32x4_t aop[KSB];
        auto mfma_half = [&](AccT(&acc)[H], int q0) {
#pragma unroll
          for (int i = 0; i < H; i++) acc[i] = AccT{0, 0, 0, 0};
#pragma unroll
          for (int c = 0; c < KSB; c++)
#pragma unroll
            for (int i = 0; i < H; i++) acc[i] = ChunkMfma<DT>::run(aop[c], qreg[q0 + i][c], acc[i]);
        };
        auto fold_half = [&](int t, const AccT(&acc)[H], int q0) {
          const int row0 = blk * BLK_ROWS + t * 16 + 4 * g;
#pragma unroll
          for (int i = 0; i < H; i++) {
            if constexpr (ARG) {
#pragma unroll
              for (int r = 0; r < 4; r++) {
                if (acc[i][r] > m[q0 + i]) {
                  m[q0 + i] = acc[i][r];
                  arg[q0 + i] = row0 + r;
                }
              }
            } else {
              m[q0 + i] = __builtin_fmaxf(m[q0 + i], max4(acc[i]));
            }
          }
        };
        auto interleave_half = [&]() {
          constexpr int VPM = ((ARG ? 12 : 4) + KSB - 1) / KSB;
#pragma unroll
          for (int i = 0; i < H * KSB; i++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
          }
        };
        auto read_tile = [&](int t) {
#pragma unroll
          for (int c = 0; c < KSB; c++) aop[c] = read_a(t, c);
        };
        // With the argmax, the next tile's A operands are read as soon as this tile's second
        // half has taken them: chunk c's read follows chunk c's MFMAs, inside the interleave,
        // and the first half's fold covers the LDS latency. Forward with argmax at the ColPali
        // training shape: 2.312-2.360 -> 2.264-2.289 ms. The several-query instance keeps the
        // later read: with it, it would spill.
        auto interleave_half_reads = [&]() {
          constexpr int VPM = ((ARG ? 12 : 4) + KSB - 1) / KSB;
#pragma unroll
          for (int c = 0; c < KSB; c++) {
#pragma unroll
            for (int i = 0; i < H; i++) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        };
        read_tile(0);
        mfma_half(accA, 0);
        int t = 0;
        for (; t + 1 < ntiles; t++) {
          mfma_half(accB, H);
          if constexpr (ARG) {
            read_tile(t + 1);
            fold_half(t, accA, 0);
            interleave_half_reads();
          } else {
            fold_half(t, accA, 0);
            interleave_half();
            read_tile(t + 1);
          }
          mfma_half(accA, 0);
          fold_half(t, accB, H);
          interleave_half();
        }
        mfma_half(accB, H);
        fold_half(t, accA, 0);
        fold_half(t, accB, H);
      } else if constexpr (!I8) {
        // The next tile's A operands are read once this tile's MFMAs are issued, so the LDS
        // latency runs under the last MFMAs and the fold instead of stalling the next tile
        // (scheduling barriers keep that order). Measured at the ColPali shape: 1.795-1.807
        // -> 1.776-1.785 ms; reading them before this tile's MFMAs instead (both sets live,
        // 254 VGPRs) was 2% slower than reading them at the tile's start. (The INT8
        // instances here, the widest slices, keep the loop below: one of them would spill.)
        u32x4_t aop[KSB];
#pragma unroll
        for (int c = 0; c < KSB; c++) aop[c] = read_a(0, c);
        for (int t = 0; t < ntiles; t++) {
          AccT acc[QBW];
          scale_tile(t);
          mfma_tile(acc, aop);
          const int tn = t + 1 < ntiles ? t + 1 : t;
#pragma unroll
          for (int c = 0; c < KSB; c++) aop[c] = read_a(tn, c);
          fold(t, acc);
          __builtin_amdgcn_sched_group_barrier(0x008, QBW * KSB, 0);  // the MFMAs,
          __builtin_amdgcn_sched_group_barrier(0x100, KSB, 0);        // the next A reads,
          __builtin_amdgcn_sched_group_barrier(0x002, 4 * QBW, 0);    // then the fold
        }
      } else {
        for (int t = 0; t < ntiles; t++) {
          u32x4_t aop[KSB];
#pragma unroll
          for (int c = 0; c < KSB; c++) aop[c] = read_a(t, c);
          AccT acc[QBW];
          scale_tile(t);
          mfma_tile(acc, aop);
          fold(t, acc);
        }
      }
    }

    if (BATCH && doc_end && local) {
      if (defer) {
        pend_epi = true;
        pend_epi_b = b;
        pend_empty = empty;
      } else {
        doc_epilogue(b, empty);
      }
    } else if (doc_end) {
      // Each lane adds its maxima over consecutive blocks of one query in double; where the
      // query changes (wave-uniform) the lanes reduce and the segment's sum goes to LDS slot
      // w * QBW + (first block of the segment). A query then adds its segments in order.
      double s = 0.0;
      int seg_q = blk_q[0], seg_k = uniform(w * QBW);
      auto flush = [&]() {
        s = sum_row16(s);
        if (lane == 0) part_lds[seg_k] = s;
        s = 0.0;
      };
#pragma unroll
      for (int qb = 0; qb < QBW; qb++) {
        float v = m[qb];
        int j = arg[qb];
        // combine the four row groups: larger value wins, equal values keep the lower row
        if constexpr (ARG) {
          // through LDS-routed shuffles: the register-pair form needs registers the widest
          // INT8 instance does not have, and this runs once per document
#pragma unroll
          for (int sh = 16; sh <= 32; sh <<= 1) {
            const float ov = __shfl_xor(v, sh);
            const int oj = __shfl_xor(j, sh);
            if (ov > v || (ov == v && oj < j)) {
              v = ov;
              j = oj;
            }
          }
        } else {
          v = max_row_groups(v);
        }
        if constexpr (!BATCH) {
          // a single query: token qi
          const int qi = q_base + qb * 16 + r16;
          if (qi < q_len) {
            if (!empty) s += (double)v;
            if constexpr (ARG) {
              if (g == 0) {
                a.tok_max[b * q_len + qi] = empty ? -__builtin_inff() : v;
                a.tok_arg[b * q_len + qi] = empty ? -1 : j;
              }
            }
          }
        } else {
          const int qq = blk_q[qb];
          if (qq != seg_q) {
            flush();
            seg_q = qq;
            seg_k = uniform(w * QBW + qb);
          }
          if (((real_bits >> qb) & 1u) && !empty) s += (double)v;
        }
        m[qb] = -__builtin_inff();
        arg[qb] = -1;
      }
      flush();
      __syncthreads();  // wave-uniform and the same in every wave
      if constexpr (!BATCH) {
        if (threadIdx.x == 0) {  // a single query: one segment per wave
          double tot = 0.0;
          for (int k = 0; k < NW; k++) tot += part_lds[k * QBW];
          a.out[b] = empty ? -__builtin_inff() : (float)tot;
        }
      } else {
        const int bpq = q_pad / 16;
        for (int q = threadIdx.x; q < a.n_q; q += TILED_THREADS) {
          double tot = 0.0;
          for (int k = q * bpq; k < (q + 1) * bpq; k++)
            if (k == q * bpq || k % QBW == 0) tot += part_lds[k];
          a.out[(int64_t)q * a.n_docs + b] = empty ? -__builtin_inff() : (float)tot;
        }
      }
    }
    buf ^= 1;
  }
  if constexpr (BATCH) {
    if (local) {
      if (pend_epi) doc_epilogue(pend_epi_b, pend_empty);
      local_store();
    }
  }
}

}  // namespace maxsim
