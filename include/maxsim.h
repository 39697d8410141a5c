/*
 * libmaxsim -- late-interaction MaxSim scoring on AMD Instinct MI355X (gfx950).
 *
 * The operation (TileMaxSim deep reading, section 1; Flash-MaxSim abstract and
 * Figure 1): for one query of q_len tokens q_i and each document b of len_b
 * tokens d_j,
 *
 *     out[b] = sum_{i < q_len}  max_{j < len_b}  <q_i, d_j>
 *
 * one fp32 score per (query, document) pair. The query-token x document-token
 * similarity matrix is never written to memory: each document is read from HBM
 * once, the tile products run on the matrix cores with fp32 accumulation, the
 * running maxima stay in registers and only the scalar score is stored.
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers owned by the caller. The library
 *    allocates nothing, keeps no per-call state and never reads device memory
 *    on the host. Work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream) and results are valid once that stream has synchronised.
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check returns a negative maxsim_status and enqueues nothing. A call with
 *    n_docs == 0 returns MAXSIM_OK and enqueues nothing (maxsim_backward with dQ
 *    set, which writes zeros to dQ, is the one exception).
 *  - Contents are not checked: malformed doc_offsets (decreasing, or past the
 *    token array), NaN or Inf inputs give undefined scores.
 *  - Storage is row-major and densely packed. Q, D, codes and tables must be
 *    16-byte aligned; out, scales and offsets naturally aligned.
 *  - An empty document (length 0) scores -inf (a max over no tokens).
 *  - Thread-safe; calls on different streams may overlap.
 */
#ifndef MAXSIM_H
#define MAXSIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage formats of Q and D for the dense entry points. */
enum maxsim_dtype {
  MAXSIM_BF16 = 0, /* bfloat16 */
  MAXSIM_FP16 = 1, /* IEEE binary16 */
  MAXSIM_FP32 = 2  /* IEEE binary32; full-precision products (no reduced-precision path) */
};

enum maxsim_status {
  MAXSIM_OK = 0,
  MAXSIM_ERR_NULL = -1,        /* a required pointer is NULL */
  MAXSIM_ERR_SHAPE = -2,       /* a size is out of range */
  MAXSIM_ERR_DTYPE = -3,       /* unknown dtype */
  MAXSIM_ERR_ALIGN = -4,       /* a pointer is not aligned as required */
  MAXSIM_ERR_UNSUPPORTED = -5, /* valid, but no kernel for this combination */
  MAXSIM_ERR_LAUNCH = -6,      /* the HIP runtime refused the launch */
  MAXSIM_ERR_DEVICE = -7,      /* no usable gfx950 device is current */
  MAXSIM_ERR_SCRATCH = -8      /* needs more than the library's static scratch memory */
};

/* Limits checked by every entry point. */
#define MAXSIM_MAX_Q_LEN 1024 /* query tokens (ColPali-shaped queries: Flash-MaxSim Figure 2) */
#define MAXSIM_MIN_D 32
#define MAXSIM_MAX_D 1024 /* d % 32 == 0 (TileMaxSim deep reading, section 2 item (2): d = 64..768) */

/*
 * Variable-length (padding-free) documents in CSR form (Flash-MaxSim
 * abstract: variable-length scoring; TileMaxSim deep reading, section 6:
 * packed documents).
 *   Q           [q_len][d] in `dtype`, 1 <= q_len <= MAXSIM_MAX_Q_LEN
 *   D           [doc_offsets[n_docs]][d] in `dtype`: all document tokens, packed
 *   doc_offsets int64 [n_docs + 1]; document b is tokens [doc_offsets[b], doc_offsets[b+1]);
 *               doc_offsets[0] is normally 0 and the sequence must not decrease
 *   d           embedding dimension, a multiple of 32 in [MAXSIM_MIN_D, MAXSIM_MAX_D]
 *   out         fp32 [n_docs]
 * Up to 64 query tokens are scored by one wave per document with the whole query
 * resident (in registers, or in LDS for rows wider than 512 bytes or more than 16 query
 * registers per row, where ceil(q_len / 16) * 16 * (d * element bytes + 16) must fit in
 * 160 KiB: fp32 with 49-64 tokens and d >= 640, or 33-48 tokens and d >= 864, return
 * MAXSIM_ERR_UNSUPPORTED); longer queries (up to 1024, Flash-MaxSim Figure 2: Lq = 1024) are split
 * across the waves of a workgroup and need d * element bytes to be 64, 128, 256 or
 * 512 bytes and q_len <= 1024 * 64 / (d * element bytes), else MAXSIM_ERR_UNSUPPORTED.
 */
int maxsim_score(const void *Q, int q_len, const void *D, const int64_t *doc_offsets,
                 int64_t n_docs, int d, int dtype, float *out, void *stream);

/*
 * Fixed-length documents (TileMaxSim deep reading, section 2: documents of Nd
 * tokens; section 5: padding to a fixed Nd).
 *   D        [n_docs][nd][d] in `dtype`, nd >= 1
 *   doc_lens nullable int32 [n_docs]: valid tokens of each document; tokens
 *            j >= doc_lens[b] are padding and never affect the score. Values are
 *            clamped to [0, nd]. NULL means every document has nd valid tokens.
 *   other arguments as for maxsim_score.
 */
int maxsim_score_fixed(const void *Q, int q_len, const void *D, int64_t n_docs, int nd,
                       const int32_t *doc_lens, int d, int dtype, float *out, void *stream);

/*
 * Several queries against the same documents in one pass over them (each document byte
 * read once per group of queries; TileMaxSim deep reading, section 2 item (1): tiling
 * along queries as well): out[q][b] = sum_i max_j <Q[q][i], d_j>.
 *   Q        [n_q][q_len][d] in `dtype`, n_q >= 1
 *   D, doc_offsets / nd, d, dtype  as for maxsim_score_argmax (CSR, or fixed when NULL)
 *   out      fp32 [n_q][n_docs]
 * Queries are padded to whole 16-token blocks and grouped so that a group holds at most
 * 1024 * 64 / (d * element bytes) (at most 1024) padded tokens; each group is one launch.
 * Needs d * element bytes to be 64, 128, 256 or 512, else MAXSIM_ERR_UNSUPPORTED.
 */
int maxsim_score_batch(const void *Q, int n_q, int q_len, const void *D,
                       const int64_t *doc_offsets, int64_t n_docs, int nd, int d, int dtype,
                       float *out, void *stream);

/*
 * Scores with per-token maxima and argmax, for the backward pass (Flash-MaxSim
 * abstract and page: training reuses the forward's argmax locations).
 *   Q, D, d, dtype as for maxsim_score; doc_offsets nullable: CSR as in
 *            maxsim_score, or NULL for fixed documents D [n_docs][nd][d] (nd >= 1)
 *   out      fp32 [n_docs] scores, exactly as maxsim_score / maxsim_score_fixed
 *   tok_max  fp32 [n_docs][q_len]: max_j <q_i, d_j> (the fp32 value the score sums)
 *   tok_arg  int32 [n_docs][q_len]: the lowest j whose fp32 similarity equals that
 *            maximum; an empty document gives -inf and -1.
 * Both outputs are required. Sizes supported as for maxsim_score.
 */
int maxsim_score_argmax(const void *Q, int q_len, const void *D, const int64_t *doc_offsets,
                        int64_t n_docs, int nd, int d, int dtype, float *out, float *tok_max,
                        int32_t *tok_arg, void *stream);

/*
 * Backward pass: gradients of L = sum_b grad_out[b] * out[b] given the forward argmax
 * (Flash-MaxSim abstract and page: backward through the argmax; inverse-grid CSR with
 * an atomic-free, destination-owned reduction):
 *     dD[b][j] = grad_out[b] * sum of q_i over the query tokens i with tok_arg[b][i] == j
 *                (zero where no query token chose j)
 *     dQ[i]    = sum_b grad_out[b] * D[b][tok_arg[b][i]]
 *   Q, D, doc_offsets / nd, d, dtype  as for maxsim_score_argmax
 *   tok_arg    int32 [n_docs][q_len] from maxsim_score_argmax (an entry outside
 *              [0, len_b), such as the -1 of an empty document, contributes nothing)
 *   grad_out   fp32 [n_docs]
 *   grad_dtype type of dQ and dD: MAXSIM_FP32, or dtype itself (each value rounded
 *              once, to nearest even, from its fp32 sum)
 *   dQ         nullable [q_len][d] in grad_dtype: written when set (needs the workspace);
 *              with n_docs == 0 it is set to zero (the one launch a call with no
 *              documents enqueues; D, tok_arg and grad_out may then be NULL)
 *   dD         nullable [tokens][d] in grad_dtype: every row of every document is
 *              written when set; rows of tokens outside all documents are left untouched
 *   workspace  device buffer of at least maxsim_backward_workspace_size(q_len, d,
 *              n_docs) bytes, 16-byte aligned, when dQ is set (NULL otherwise); its
 *              contents on entry do not matter
 * The result does not depend on the run: every output element has one writer and a
 * fixed summation order. dQ and dD are 16-byte aligned.
 */
int maxsim_backward(const void *Q, int q_len, const void *D, const int64_t *doc_offsets,
                    int64_t n_docs, int nd, int d, int dtype, const int32_t *tok_arg,
                    const float *grad_out, void *dQ, void *dD, int grad_dtype, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Workspace bytes maxsim_backward needs for dQ (0 for invalid sizes or n_docs == 0). */
size_t maxsim_backward_workspace_size(int q_len, int d, int64_t n_docs);

/*
 * INT8 x INT8 scoring with per-token fp32 scales (Flash-MaxSim abstract:
 * INT8xINT8 quantisation). With dot_ij the exact int32 dot product of the
 * stored int8 tokens, the scaled similarity is
 *     v_ij = fl32( fl32(dot_ij) * fl32(q_scale[i] * d_scale[j]) )
 * (round to nearest even, each product rounded once); out[b] = sum_i max_j v_ij.
 *   Q        int8 [q_len][d];  q_scale fp32 [q_len]
 *   D        int8 [tokens][d]; d_scale fp32 [tokens]
 *   doc_offsets  nullable: CSR as in maxsim_score; NULL means fixed documents of
 *            nd tokens each (tokens = n_docs * nd)
 *   d        64, 128, 256 or 512 (other multiples of 64 return MAXSIM_ERR_UNSUPPORTED)
 *   tok_max  nullable fp32 [n_docs][q_len]: max_j v_ij per query token (bit-exact)
 *   tok_arg  nullable int32 [n_docs][q_len]: the j attaining it, lowest j on ties,
 *            -1 for an empty document. tok_max and tok_arg are both NULL or both set.
 */
int maxsim_score_i8(const int8_t *Q, const float *q_scale, int q_len, const int8_t *D,
                    const float *d_scale, const int64_t *doc_offsets, int64_t n_docs, int nd,
                    int d, float *out, float *tok_max, int32_t *tok_arg, void *stream);

/*
 * Per-query product-quantisation distance tables (TileMaxSim deep reading,
 * section 2 item (3)):  T[i][m][k] = sum_{t < dsub} Q[i][m*dsub + t] * C[m][k][t]
 *   Q  [q_len][M*dsub] in `dtype`
 *   C  fp32 [M][K][dsub] codebook
 *   T  fp32 [q_len][M][K] (output, caller-allocated: q_len*M*K*4 bytes)
 *   Supported: K == 256, M*dsub a multiple of 32 in [MAXSIM_MIN_D, MAXSIM_MAX_D], dsub <= 32.
 */
int maxsim_pq_tables(const void *Q, int q_len, int dtype, const float *C, int M, int K, int dsub,
                     float *T, void *stream);

/*
 * Fused PQ lookup scoring (TileMaxSim deep reading, section 2 item (3)): token
 * j's similarity to query token i is sum_m T[i][m][codes[j][m]], then max over
 * j and sum over i as above. Codes are never decompressed to vectors.
 *   T      fp32 [q_len][M][K] from maxsim_pq_tables
 *   codes  uint8 [tokens][M]
 *   doc_offsets nullable: CSR, or NULL for fixed documents of nd tokens
 *   Supported: K == 256, M == 16, q_len <= 64.
 */
int maxsim_score_pq(const float *T, int q_len, int M, int K, const uint8_t *codes,
                    const int64_t *doc_offsets, int64_t n_docs, int nd, float *out, void *stream);

/*
 * Top-k selection after scoring (the stage that hands the best documents on): for each of
 * `rows` rows of n scores (a [rows][n] array such as the output of maxsim_score_batch),
 * the k entries that come first in the order score descending, document index ascending,
 * in that order. The selection is exact and the same on every run (no atomics).
 *   scores     fp32 [rows][n]; 1 <= n < 2^31, 1 <= rows <= 65535; NaN is not ordered
 *   k          1 <= k <= 1024; if k > n the tail holds -inf and index -1
 *   out_scores fp32 [rows][k]; out_index int32 [rows][k]
 *   workspace  device buffer of at least maxsim_topk_workspace_size(n, rows, k) bytes,
 *              8-byte aligned (NULL allowed when that size is 0)
 */
int maxsim_topk(const float *scores, int64_t n, int rows, int k, float *out_scores,
                int32_t *out_index, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes maxsim_topk needs (0 when n fits one 2048-entry chunk or on bad sizes). */
size_t maxsim_topk_workspace_size(int64_t n, int rows, int k);

/*
 * maxsim_topk for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same selection and
 * the same results, with the workspace taken from a static device array inside the
 * library (maxsim_topk_scratch_bytes(), 8 MiB; each GPU the library runs on holds its own
 * copy until the process ends). Allocates nothing.
 *   Arguments as for maxsim_topk, without the workspace.
 *   Returns MAXSIM_ERR_SCRATCH when maxsim_topk_workspace_size(n, rows, k) exceeds the
 *   static array (for k <= 128: rows * (runs of 2048 scores + runs of the first merge) of
 *   1 KiB each, 8192 in all).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and give undefined results.
 */
int maxsim_topk_no_alloc(const float *scores, int64_t n, int rows, int k, float *out_scores,
                         int32_t *out_index, void *stream);

/* Bytes of the static scratch array maxsim_topk_no_alloc uses on each GPU. */
size_t maxsim_topk_scratch_bytes(void);

/* Static description of a status code. */
const char *maxsim_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int maxsim_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAXSIM_H */
