"""GPU parity of several queries scored in one pass over the documents
(maxsim_score_batch): each (query, document) score against the oracle's single-query score
of that query (|delta| <= 1e-4), with queries padded inside the kernel, groups of queries
split across launches, CSR documents with empty ones, and a single query bit-identical to
the single-query entry point. Up to 16 query blocks of two-byte rows of 128 or 256 bytes
run on the one-wave-per-document kernel with the queries in LDS; the rest on the
query-tiled kernel."""
import numpy as np
import pytest

import gen
import oracle
from gpu_util import TOL, compare, ms, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ms()


def queries(seed, n_q, q_len, d, dtype):
    Q = gen.tokens(seed, gen.S_QUERY, 0, n_q * q_len, d, dtype)
    return Q.reshape(n_q, q_len, d)


def gpu_batch(Q, D, dtype, offsets=None):
    import torch
    off = None if offsets is None else torch.from_numpy(offsets).cuda()
    out = ms().maxsim_score_batch(gen.to_device(Q, dtype), gen.to_device(D, dtype), off)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


CASES = [  # n_q, q_len, d, dtype, layout
    # one-wave-per-document kernel (at most 16 blocks, rows of 128 or 256 bytes)
    (4, 32, 128, "bf16", "fixed"),
    (3, 7, 64, "fp16", "fixed"),      # padding inside every query; 3 blocks and a zero one
    (8, 32, 128, "bf16", "fixed"),    # 16 blocks, 2 per query
    (16, 16, 128, "bf16", "csr"),     # 1 block per query
    (4, 64, 128, "bf16", "csr"),      # 4 blocks per query
    (7, 32, 128, "bf16", "csr"),      # 14 blocks
    (8, 30, 128, "bf16", "csr"),      # padding tokens in every query
    (2, 100, 128, "bf16", "csr"),     # 7-block queries
    (16, 1, 128, "fp16", "csr"),      # one-token queries
    (2, 128, 64, "fp16", "fixed"),    # 8-block queries, 128-byte rows
    (5, 48, 128, "bf16", "fixed"),    # 15 blocks and a zero one
    # query-tiled kernel
    (32, 32, 128, "bf16", "fixed"),   # 1024 tokens: one launch
    (40, 32, 128, "bf16", "csr"),     # two launches
    (5, 100, 128, "bf16", "csr"),     # 112-token padded queries, 9 per launch
    (2, 64, 256, "bf16", "fixed"),
    (6, 33, 128, "fp32", "fixed"),    # fp32 rows of 512 B: 512 tokens per launch
    (17, 1, 128, "bf16", "csr"),      # one-token queries
    (3, 1024, 128, "bf16", "fixed"),  # one query per launch
    # 4 or 8 query blocks per wave, queries of 1, 2 or 4 blocks: the row groups exchange
    # their maxima so that each sums one block (the four-block document end)
    (8, 32, 256, "bf16", "fixed"),    # 4 blocks per wave, 2 per query
    (16, 16, 128, "fp32", "csr"),     # 4 blocks per wave, 1 per query
    (4, 64, 256, "bf16", "csr"),      # 4 blocks per wave, 4 per query
    (7, 32, 256, "fp16", "csr"),      # the last wave's second query is padding
    (64, 16, 128, "bf16", "fixed"),   # 8 blocks per wave, 1 per query
    (16, 64, 128, "fp16", "csr"),     # 8 blocks per wave, 4 per query
    (29, 32, 128, "bf16", "csr"),     # 8 blocks per wave, padding queries in the last wave
    (8, 30, 128, "fp32", "csr"),      # 4 blocks per wave: padding tokens in every query
    (32, 20, 128, "bf16", "fixed"),   # 8 blocks per wave: padding tokens in every query
]


@pytest.mark.parametrize("n_q,q_len,d,dtype,layout", CASES)
def test_batch_matches_single_query_oracle(n_q, q_len, d, dtype, layout):
    say(f"case: batch n_q={n_q} q_len={q_len} d={d} {dtype} {layout}")
    seed = 700 + n_q + q_len + d
    Q = queries(seed, n_q, q_len, d, dtype)
    if layout == "fixed":
        c = gen.fixed_corpus(seed, 37, 1, 90, d, dtype)
        want = oracle.maxsim_batch(Q, c.D, dtype)
        got = gpu_batch(Q, c.D, dtype)
    else:
        lens = np.concatenate([[0, 1, 130, 0, 16, 17], gen.lengths(seed, 40)])
        c = gen.csr_corpus(seed, len(lens), 1, d, dtype, lens=lens)
        want = oracle.maxsim_batch(Q, c.D, dtype, offsets=c.offsets)
        got = gpu_batch(Q, c.D, dtype, c.offsets)
    assert got.shape == (n_q, want.shape[1])
    compare(got.ravel(), want.ravel(), what=f"batch n_q={n_q} q_len={q_len}")


def test_batch_more_documents_than_workgroups():
    """600 CSR documents (empty ones, one-token ones, and ones spanning two 32 KiB blocks)
    for 32 queries of 32 tokens: every workgroup walks several documents, so the waves that
    take their document-end reductions after the next block's barrier do so inside the
    block loop as well as after it."""
    n_q, q_len, d, dtype = 32, 32, 64, "bf16"
    say(f"case: batch n_q={n_q} q_len={q_len} d={d} over 600 CSR documents")
    seed = 741
    Q = queries(seed, n_q, q_len, d, dtype)
    lens = gen.lengths(seed, 600, median=20.0, sigma=0.8, lo=1, hi=300)
    lens[::37] = 0
    lens[5::53] = 300  # two blocks of 256 rows
    c = gen.csr_corpus(seed, len(lens), 1, d, dtype, lens=lens)
    want = oracle.maxsim_batch(Q, c.D, dtype, offsets=c.offsets)
    got = gpu_batch(Q, c.D, dtype, c.offsets)
    compare(got.ravel(), want.ravel(), what="batch over 600 documents")


@pytest.mark.parametrize("n_q,q_len,d,nd", [(8, 32, 64, None), (4, 64, 128, None),
                                            (4, 32, 128, 8), (8, 32, 64, 8)])
def test_dense_batch_many_documents_per_wave(n_q, q_len, d, nd):
    """The one-wave-per-document kernel over many documents: 600 CSR documents (empty ones,
    one-token ones, lengths around the 64-token groups, up to 300 tokens), or 20000 fixed
    documents of 8 tokens, enough for one contiguous range per wave."""
    dtype = "bf16"
    seed = 760 + n_q + q_len + d
    Q = queries(seed, n_q, q_len, d, dtype)
    if nd is None:
        say(f"case: dense batch n_q={n_q} q_len={q_len} d={d} over 600 CSR documents")
        lens = gen.lengths(seed, 600, median=40.0, sigma=0.9, lo=1, hi=300)
        lens[::37] = 0
        lens[1:40:8] = [63, 64, 65, 128, 129]
        c = gen.csr_corpus(seed, len(lens), 1, d, dtype, lens=lens)
        want = oracle.maxsim_batch(Q, c.D, dtype, offsets=c.offsets)
        got = gpu_batch(Q, c.D, dtype, c.offsets)
    else:
        say(f"case: dense batch n_q={n_q} q_len={q_len} d={d} over 20000 fixed documents")
        c = gen.fixed_corpus(seed, 20000, 1, nd, d, dtype)
        want = oracle.maxsim_batch(Q, c.D, dtype)
        got = gpu_batch(Q, c.D, dtype)
    compare(got.ravel(), want.ravel(), what=f"dense batch n_q={n_q} q_len={q_len} d={d}")


@pytest.mark.parametrize("q_len", [100, 512])
def test_single_query_batch_is_bit_identical(q_len):
    """n_q = 1 runs the single-query kernels, as maxsim_score_fixed does."""
    import torch
    say(f"case: batch of one, q_len={q_len}")
    c = gen.fixed_corpus(720 + q_len, 20, q_len, 150, 128, "bf16")
    Q, D = gen.to_device(c.Q, "bf16"), gen.to_device(c.D, "bf16")
    one = ms().maxsim_score_fixed(Q, D)
    batch = ms().maxsim_score_batch(Q.unsqueeze(0).contiguous(), D)
    torch.cuda.synchronize()
    assert torch.equal(one, batch[0])


def test_batch_unsupported_row_width_raises():
    say("case: batch d=768 bf16 (no kernel)")
    Q = queries(730, 2, 8, 768, "bf16")
    c = gen.fixed_corpus(730, 3, 1, 16, 768, "bf16")
    with pytest.raises(Exception):
        gpu_batch(Q, c.D, "bf16")
