"""GPU parity of the product-quantisation path: table build and fused lookup scoring,
against the oracle with the same codebook and codes (|delta| <= 1e-3)."""
import numpy as np
import pytest

import gen
import oracle
from gpu_util import PQ_TOL, compare, ms, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ms()


def gpu_tables(Q, dtype, C):
    import torch
    T = ms().maxsim_pq_tables(gen.to_device(Q, dtype), torch.from_numpy(C).cuda())
    torch.cuda.synchronize()
    return T


def gpu_pq(T, codes, offsets=None, nd=0):
    import torch
    off = None if offsets is None else torch.from_numpy(offsets).cuda()
    out = ms().maxsim_score_pq(T, torch.from_numpy(codes).cuda(), off, nd=nd)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("dsub,M", [(8, 16), (4, 16), (2, 16), (16, 8)])
def test_tables(dtype, dsub, M):
    say(f"case: PQ tables {dtype} M={M} dsub={dsub}")
    C = gen.codebook(41, M, 256, dsub)
    Q = gen.tokens(41, gen.S_QUERY, 0, 32, M * dsub, dtype)
    want = oracle.pq_tables(Q, dtype, C)
    got = gpu_tables(Q, dtype, C).cpu().numpy().astype(np.float64)
    err = np.abs(got - want).max()
    say(f"  tables max |gpu - oracle| = {err:.2e}")
    assert err <= 1e-6


@pytest.mark.parametrize("q_len", [1, 7, 8, 9, 32, 64])
@pytest.mark.parametrize("n_docs", [1, 63, 64, 65, 200])
def test_score_fixed(q_len, n_docs):
    say(f"case: PQ fixed q_len={q_len} n_docs={n_docs} nd=128")
    C = gen.codebook(42)
    Q = gen.tokens(42, gen.S_QUERY, 0, q_len, 128, "bf16")
    codes = gen.codes(42, n_docs * 128)
    T = gpu_tables(Q, "bf16", C)
    want = oracle.maxsim_pq(oracle.pq_tables(Q, "bf16", C), codes, nd=128)
    compare(gpu_pq(T, codes, nd=128), want, tol=PQ_TOL, what=f"PQ fixed q={q_len} B={n_docs}")


def test_score_uses_given_tables_exactly():
    """Scores computed from the oracle's tables (rounded to fp32) match the oracle run on
    the same fp32 tables: only the fp32 additions differ."""
    import torch
    say("case: PQ scorer on oracle tables")
    C = gen.codebook(43)
    Q = gen.tokens(43, gen.S_QUERY, 0, 32, 128, "bf16")
    T32 = oracle.pq_tables(Q, "bf16", C).astype(np.float32)
    codes = gen.codes(43, 300 * 40)
    want = oracle.maxsim_pq(T32.astype(np.float64), codes, nd=40)
    got = gpu_pq(torch.from_numpy(T32).cuda(), codes, nd=40)
    compare(got, want, tol=1e-4, what="PQ on fixed tables")


def test_score_csr_ragged_with_empty_docs():
    lens = np.concatenate([[0, 1, 512, 0, 128, 129, 7],
                           gen.lengths(44, 250)]).astype(np.int64)
    say(f"case: PQ CSR {len(lens)} docs incl. empty")
    off = gen.csr_offsets(lens)
    C = gen.codebook(44)
    Q = gen.tokens(44, gen.S_QUERY, 0, 32, 128, "bf16")
    codes = gen.codes(44, int(off[-1]))
    T = gpu_tables(Q, "bf16", C)
    want = oracle.maxsim_pq(oracle.pq_tables(Q, "bf16", C), codes, offsets=off)
    got = gpu_pq(T, codes, offsets=off)
    assert np.all(np.isneginf(got[lens == 0]))
    compare(got, want, tol=PQ_TOL, what="PQ CSR")


# The scorer gives each workgroup (one per CU) a contiguous range of documents, balanced by
# tokens for CSR corpora, cut into equal chunks of at most 512 documents, and stages each
# table slice once for up to 4 of its chunks. On 256 CUs: 16384 and 16385 documents give one
# chunk of 64-65 documents per workgroup, 40000 give 156-157, 140000 give two chunks of about
# 273, and 600000 give five chunks of about 469 (two groups of chunks per slice staging).
@pytest.mark.parametrize("n_docs,nd", [(16384, 9), (16385, 9), (40000, 9), (140000, 2),
                                       (600000, 1)])
def test_score_fixed_many_documents_per_chunk(n_docs, nd):
    say(f"case: PQ fixed n_docs={n_docs} nd={nd} (documents per chunk > 1)")
    C = gen.codebook(46)
    Q = gen.tokens(46, gen.S_QUERY, 0, 32, 128, "bf16")
    codes = gen.codes(46, n_docs * nd)
    T = gpu_tables(Q, "bf16", C)
    want = oracle.maxsim_pq(oracle.pq_tables(Q, "bf16", C), codes, nd=nd)
    compare(gpu_pq(T, codes, nd=nd), want, tol=PQ_TOL, what=f"PQ fixed B={n_docs} nd={nd}")


@pytest.mark.parametrize("n_docs,max_len", [(40000, 24), (200000, 3)])
def test_score_csr_many_documents_per_chunk(n_docs, max_len):
    """Many short CSR documents (empty ones among them): token-balanced workgroup ranges of
    about 156 (40000 documents) or 780 (200000, two chunks per workgroup) documents whose
    token runs cross many document boundaries."""
    lens = np.random.default_rng(47 + max_len).integers(0, max_len + 1, size=n_docs).astype(np.int64)
    lens[:5] = [0, 0, max_len, 1, 0]
    say(f"case: PQ CSR {len(lens)} short docs (at most {max_len} tokens)")
    off = gen.csr_offsets(lens)
    C = gen.codebook(47)
    Q = gen.tokens(47, gen.S_QUERY, 0, 32, 128, "bf16")
    codes = gen.codes(47, int(off[-1]))
    T = gpu_tables(Q, "bf16", C)
    want = oracle.maxsim_pq(oracle.pq_tables(Q, "bf16", C), codes, offsets=off)
    got = gpu_pq(T, codes, offsets=off)
    assert np.all(np.isneginf(got[lens == 0]))
    compare(got, want, tol=PQ_TOL, what=f"PQ CSR {n_docs} short docs")


def test_planted_docs_rank_first_after_encoding():
    """Planted near-duplicates stay on top after nearest-centroid PQ encoding."""
    say("case: PQ planted top-k")
    c = gen.csr_corpus(45, 400, 32, 128, "bf16", n_plant=5)
    x = (c.D.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    C = gen.codebook(45)
    codes = gen.pq_encode(x, C)
    T = gpu_tables(c.Q, "bf16", C)
    got = gpu_pq(T, codes, offsets=c.offsets)
    want = oracle.maxsim_pq(oracle.pq_tables(c.Q, "bf16", C), codes, offsets=c.offsets)
    compare(got, want, tol=PQ_TOL, what="PQ planted")
    top = np.lexsort((np.arange(len(got)), -got))[:5]
    assert set(top.tolist()) == set(c.planted.tolist())


@pytest.mark.parametrize("q_len", [5, 20, 32, 64])
@pytest.mark.parametrize("layout", ["csr", "fixed"])
def test_score_several_token_capped_chunks(layout, q_len):
    """Workgroup ranges of about 12.5K tokens: with a chunk cap of 6144 tokens (the
    MAXSIM_PQ_CHUNK_TOK knob, read at every call) three chunks each, so the slices are walked
    up, down and up again (the slice at each chunk boundary is not staged again) with 1, 3, 4
    or 8 slices of 8 query tokens; empty CSR documents among them. Without the cap (the
    default) the same corpora take one chunk per workgroup, also checked, and both give the
    same scores bit for bit (each document's arithmetic does not depend on the chunking)."""
    import os
    rng = np.random.default_rng(60 + q_len)
    if layout == "csr":
        lens = rng.integers(0, 161, size=40000).astype(np.int64)
        lens[::97] = 0
        off = gen.csr_offsets(lens)
        n_tok, nd = int(off[-1]), 0
    else:
        off, nd = None, 80
        n_tok = 40000 * nd
    say(f"case: PQ {layout} q_len={q_len}, {n_tok} tokens, several chunks per workgroup")
    C = gen.codebook(60)
    Q = gen.tokens(60, gen.S_QUERY, 0, q_len, 128, "bf16")
    codes = gen.codes(60 + q_len, n_tok)
    T = gpu_tables(Q, "bf16", C)
    Th = oracle.pq_tables(Q, "bf16", C)
    want = oracle.maxsim_pq(Th, codes, offsets=off) if off is not None else \
        oracle.maxsim_pq(Th, codes, nd=nd)
    saved = os.environ.get("MAXSIM_PQ_CHUNK_TOK")
    try:
        os.environ["MAXSIM_PQ_CHUNK_TOK"] = "6144"
        got = gpu_pq(T, codes, offsets=off, nd=nd)
        os.environ["MAXSIM_PQ_CHUNK_TOK"] = "0"
        whole = gpu_pq(T, codes, offsets=off, nd=nd)
    finally:
        if saved is None:
            os.environ.pop("MAXSIM_PQ_CHUNK_TOK", None)
        else:
            os.environ["MAXSIM_PQ_CHUNK_TOK"] = saved
    compare(got, want, tol=PQ_TOL, what=f"PQ {layout} q_len={q_len} several chunks")
    assert np.array_equal(got, whole)
