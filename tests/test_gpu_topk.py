"""GPU parity of top-k selection (maxsim_topk): on a given fp32 score array the selection is
exact, so values must be bit-identical and indices identical to the oracle's order (score
descending, index ascending), including ties, -inf entries, several rows, k > n, and sizes
that need one to several selection levels. End to end (scores from the GPU, the oracle ranking
its own float64 scores), the top-k must agree except where oracle scores tie within the
tolerance."""
import numpy as np
import pytest

import gen
import oracle
from gpu_util import TOL, gpu_scores_fixed, ms, say, topk_agree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ms()


def gpu_topk(S, k):
    import torch
    v, i = ms().maxsim_topk(torch.from_numpy(np.ascontiguousarray(S)).cuda(), k)
    torch.cuda.synchronize()
    return v.cpu().numpy(), i.cpu().numpy().astype(np.int64)


def scores_with_ties(seed, rows, n):
    rng = np.random.default_rng(seed)
    S = (rng.integers(-2000, 2000, size=(rows, n)) / 64.0).astype(np.float32)  # many ties
    S[rng.random((rows, n)) < 0.01] = -np.inf
    return S


# k <= 128 takes the run path (pass 1 over chunks of 2048, merges of up to 64 runs): 2048 and
# 2049 scores are one and two chunks; 131072 / 131073 scores make 64 / 65 runs, one and two
# merge passes; 5M scores make 2442 runs, two merge passes. k > 128 takes the LDS levels.
@pytest.mark.parametrize("n,k", [(1, 1), (5, 3), (100, 100), (2047, 10), (2048, 1024), (2049, 1024),
                                 (100_000, 10), (100_000, 100), (100_000, 1024), (1_000_000, 100),
                                 (5_000_000, 1000), (30, 64), (2048, 128), (2049, 128),
                                 (131_072, 128), (131_073, 100), (5_000_000, 100), (100_000, 129),
                                 (4096, 1), (300, 128)])
def test_topk_exact(n, k):
    say(f"case: top-{k} of {n}")
    S = scores_with_ties(800 + n % 997 + k, 1, n)[0]
    v, i = gpu_topk(S, k)
    wv, wi = oracle.topk(S, k)
    assert np.array_equal(i, wi[0]), (np.flatnonzero(i != wi[0])[:5])
    assert np.array_equal(v.view(np.uint32), wv[0].view(np.uint32))


@pytest.mark.parametrize("rows,n,k", [(3, 5000, 50), (32, 100_000, 100), (7, 2048, 1),
                                      (5, 200_000, 128), (4, 3000, 200)])
def test_topk_rows(rows, n, k):
    say(f"case: top-{k} of {rows} rows x {n}")
    S = scores_with_ties(850 + rows, rows, n)
    v, i = gpu_topk(S, k)
    wv, wi = oracle.topk(S, k)
    assert np.array_equal(i, wi) and np.array_equal(v.view(np.uint32), wv.view(np.uint32))


def test_topk_all_equal_scores_take_lowest_indices():
    say("case: top-100 of 50000 equal scores")
    S = np.full(50_000, 3.25, np.float32)
    v, i = gpu_topk(S, 100)
    assert np.array_equal(i, np.arange(100)) and np.all(v == 3.25)


def test_topk_after_scoring_planted_documents():
    """The 1000-document workload with 10 planted near-duplicates: the GPU ranking of GPU
    scores puts the planted documents first, and its top-100 agrees with the oracle's ranking
    of oracle scores except at ties within the tolerance."""
    say("case: scoring + top-k, planted corpus")
    c = gen.fixed_corpus(gen.SEEDS["C1"], 1000, 32, 128, 128, "bf16", n_plant=10)
    got = gpu_scores_fixed(c).astype(np.float32)
    want = oracle.maxsim_fixed(c.Q, c.D, "bf16")
    v, i = gpu_topk(got, 100)
    assert set(i[:10].tolist()) == set(c.planted.tolist())
    assert np.array_equal(i, oracle.topk(got, 100)[1][0])  # exact on the GPU's own scores
    topk_agree(got.astype(np.float64), want, 100, tie=2 * TOL)


@pytest.mark.parametrize("k", [100, 300])
def test_topk_signed_zeros_tie_by_index(k):
    """-0.0 and +0.0 are equal scores: their order is the index order whatever the sign, and
    the reported values keep each entry's own bits."""
    say(f"case: top-{k} with signed zeros")
    rng = np.random.default_rng(870 + k)
    n = 5000
    S = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32) * 0.0  # +-0 only
    S[rng.random(n) < 0.01] = np.float32(0.5)
    S[7], S[9] = np.float32(-0.0), np.float32(0.0)  # -0 at the lower index of a pair
    v, i = gpu_topk(S, k)
    wv, wi = oracle.topk(S, k)
    assert np.array_equal(i, wi[0]), np.flatnonzero(i != wi[0])[:5]
    assert np.array_equal(v.view(np.uint32), wv[0].view(np.uint32))
    pos7, pos9 = int(np.flatnonzero(i == 7)[0]), int(np.flatnonzero(i == 9)[0])
    assert pos7 < pos9 and np.signbit(v[pos7]) and not np.signbit(v[pos9])
