"""GPU parity of the query-tiled path: long queries (ColPali shape, up to 1024 tokens)
in bf16 / fp16 / fp32 and INT8 x INT8 with per-token scales.

INT8: per-token maxima (fp32 bits) and their argmax must equal the oracle's exactly;
scores within 1e-4."""
import numpy as np
import pytest

import gen
import oracle
from gpu_util import TOL, compare, gpu_scores_csr, gpu_scores_fixed, ms, say, topk_agree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ms()


# bf16 / fp16 queries of 65-256 tokens at d = 64 or 128 run on the document-stationary kernel
# (queries in LDS); the rest split the query across 4 waves per workgroup up to 384 tokens
# (256 at d=256 bf16) and 8 beyond: the lengths include both sides of each switch.
LONG = [(q, d) for q in (65, 100, 128, 129, 255, 257, 384, 385, 512, 1000, 1024)
        for d in (64, 128, 256) if not (d == 256 and q > 512)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("q_len,d", LONG)
def test_long_query_fixed(q_len, d, dtype):
    say(f"case: long query q_len={q_len} d={d} {dtype} B=9 Nd=300")
    c = gen.fixed_corpus(200 + q_len + d, 9, q_len, 300, d, dtype)
    compare(gpu_scores_fixed(c), oracle.maxsim_fixed(c.Q, c.D, dtype),
            what=f"q={q_len} d={d} {dtype}")


@pytest.mark.parametrize("q_len", [100, 512])
def test_long_query_fp32(q_len):
    say(f"case: long query q_len={q_len} d=128 fp32")
    c = gen.fixed_corpus(31, 7, q_len, 150, 128, "fp32")
    compare(gpu_scores_fixed(c), oracle.maxsim_fixed(c.Q, c.D, "fp32"), what="fp32 long")


def test_long_query_unsupported_shape_raises():
    say("case: q_len=1024 d=512 bf16 (no kernel)")
    c = gen.fixed_corpus(32, 2, 1024, 16, 512, "bf16")
    with pytest.raises(Exception):
        gpu_scores_fixed(c)


def test_colpali_shape_small_batch():
    """Lq = Ld = 1024, d = 128, bf16: the long-sequence shape on a handful of documents."""
    say("case: ColPali shape Lq=Ld=1024 d=128 bf16 B=12")
    c = gen.fixed_corpus(gen.SEEDS["C4"], 12, 1024, 1024, 128, "bf16")
    want = oracle.maxsim_fixed(c.Q, c.D, "bf16")
    got = gpu_scores_fixed(c)
    compare(got, want, what="ColPali bf16")
    topk_agree(got, want, 5)


def test_long_query_csr_ragged_and_empty():
    lens = np.array([0, 1, 16, 127, 128, 129, 0, 300, 1024, 5], np.int32)
    say("case: long query CSR with empty docs")
    c = gen.csr_corpus(33, len(lens), 200, 128, "bf16", lens=lens)
    got = gpu_scores_csr(c)
    assert np.all(np.isneginf(got[lens == 0]))
    compare(got, oracle.maxsim_csr(c.Q, c.D, c.offsets, "bf16"), what="long CSR")


@pytest.mark.parametrize("q_len", [100, 256, 300])
def test_long_query_doc_lens(q_len):
    """Padding past doc_lens holds large tokens that would win every max if read: on the
    document-stationary kernel (100 and 256 query tokens) and the query-tiled one (300)."""
    say(f"case: long query with doc_lens q_len={q_len}")
    c = gen.fixed_corpus(34 + q_len, 10, q_len, 200, 128, "bf16")
    lens = np.array([0, 1, 15, 16, 17, 127, 128, 129, 199, 200], np.int32)
    D = c.D.copy()
    for b in range(10):
        D[b, lens[b]:] = gen.round_bf16(np.full(128, 40.0, np.float32))
    c2 = gen.Corpus(c.seed, "bf16", 128, c.Q, D, 10, nd=200)
    compare(gpu_scores_fixed(c2, doc_lens=lens), oracle.maxsim_fixed(c.Q, c.D, "bf16", doc_lens=lens),
            what="long doc_lens")


# ---------------------------------------------------------------- INT8

def gpu_i8(c, with_tok=True):
    import torch
    m = ms()
    Q = torch.from_numpy(c.Q).cuda()
    D = torch.from_numpy(c.D).cuda()
    qs = torch.from_numpy(c.q_scale).cuda()
    ds = torch.from_numpy(np.ascontiguousarray(c.d_scale).reshape(-1)).cuda()
    off = None if c.offsets is None else torch.from_numpy(c.offsets).cuda()
    r = m.maxsim_score_i8(Q, qs, D, ds, off, with_token_max=with_tok)
    torch.cuda.synchronize()
    if with_tok:
        return (r[0].cpu().numpy().astype(np.float64), r[1].cpu().numpy(), r[2].cpu().numpy())
    return r.cpu().numpy().astype(np.float64)


def check_i8(c, what):
    want, wtm, wta = oracle.maxsim_i8(c.Q, c.q_scale, c.D, c.d_scale, c.offsets)
    got, gtm, gta = gpu_i8(c)
    compare(got, want, what=what)
    assert np.array_equal(gtm.view(np.uint32), wtm.view(np.uint32)), f"{what}: token maxima differ"
    assert np.array_equal(gta, wta), f"{what}: token argmax differs"
    # the scores-only variant gives the same scores bit for bit
    assert np.array_equal(gpu_i8(c, with_tok=False), got)


@pytest.mark.parametrize("q_len", [1, 16, 32, 100, 256, 384, 385, 1024])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_int8_fixed(q_len, d):
    say(f"case: int8 q_len={q_len} d={d} B=11 Nd=150")
    c = gen.fixed_corpus(300 + q_len + d, 11, q_len, 150, d, "i8")
    check_i8(c, f"i8 q={q_len} d={d}")


@pytest.mark.parametrize("q_len", [64, 256, 257, 512])
def test_int8_rows_of_512_bytes(q_len):
    """d = 512: 4 waves up to 256 query tokens, 8 beyond."""
    say(f"case: int8 q_len={q_len} d=512 B=7 Nd=40")
    c = gen.fixed_corpus(340 + q_len, 7, q_len, 40, 512, "i8")
    check_i8(c, f"i8 q={q_len} d=512")


def test_int8_colpali_shape():
    say("case: int8 Lq=Ld=1024 d=128 B=6")
    c = gen.fixed_corpus(gen.SEEDS["C4"], 6, 1024, 1024, 128, "i8")
    check_i8(c, "i8 ColPali")


def test_int8_csr_with_empty_docs():
    lens = np.array([0, 3, 256, 257, 0, 600, 1], np.int32)
    say("case: int8 CSR with empty docs")
    c = gen.csr_corpus(35, len(lens), 64, 128, "i8", lens=lens)
    check_i8(c, "i8 CSR")
    _, tm, ta = gpu_i8(c)
    assert np.all(np.isneginf(tm[lens == 0])) and np.all(ta[lens == 0] == -1)


@pytest.mark.parametrize("q_len", [32, 100])
def test_int8_zero_tokens(q_len):
    """Zero tokens quantise to all-zero codes with scale 0: their similarities are +0.
    A document of zero tokens, zero tokens inside a document and a zero query token, on the
    one-wave-per-document kernel (32 query tokens) and the query-tiled one (100)."""
    say(f"case: int8 zero tokens q_len={q_len}")
    c = gen.fixed_corpus(360 + q_len, 6, q_len, 70, 128, "i8")
    c.D[1] = 0
    c.d_scale[1] = 0.0
    c.D[2, 5:40] = 0
    c.d_scale[2, 5:40] = 0.0
    c.Q[3] = 0
    c.q_scale[3] = 0.0
    check_i8(c, f"i8 zero tokens q={q_len}")
    _, tm, ta = gpu_i8(c)
    assert np.all(tm[1] == 0.0) and np.all(ta[1] == 0)  # all +0: the first token
    assert np.all(tm[:, 3] >= 0.0)


def test_int8_literal_int32_maxima_and_ties():
    """Unit scales: token maxima are the int32 maxima of the dot products; duplicated
    tokens create ties that must resolve to the lowest index."""
    say("case: int8 unit scales with duplicate tokens")
    rng = np.random.default_rng(7)
    B, nd, d, q = 9, 70, 128, 40
    Q = rng.integers(-127, 128, size=(q, d)).astype(np.int8)
    D = rng.integers(-127, 128, size=(B, nd, d)).astype(np.int8)
    D[:, 50] = D[:, 3]
    D[:, 69] = D[:, 20]
    c = gen.Corpus(0, "i8", d, Q, D, B, nd=nd, q_scale=np.ones(q, np.float32),
                   d_scale=np.ones((B, nd), np.float32))
    check_i8(c, "i8 unit scales")
    _, tm, ta = gpu_i8(c)
    dots = np.einsum("ik,bjk->bij", Q.astype(np.int64), D.astype(np.int64))
    assert np.array_equal(tm, dots.max(axis=2).astype(np.float32))
    assert np.array_equal(ta, dots.argmax(axis=2))
