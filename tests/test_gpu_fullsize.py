"""Parity at the benchmark's full sizes, in the launch configuration bench.py times.

The inputs are built by bench.make_inputs (the same seeded generator and layout the
benchmark uses). The headline ColBERT workload, the CSR corpus and the PQ corpus are
checked against the oracle on every document. The other workloads are checked on
sampled documents regenerated on the host; for pool-replicated corpora every replica
must also equal its pool document bit for bit."""
import numpy as np
import pytest

import bench
import gen
import oracle
from gpu_util import PQ_TOL, TOL, compare, ms, say, topk_agree

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ms()
    yield
    torch.cuda.empty_cache()


def run(name):
    """Build the workload as bench.py does and run one step; returns (w, inputs, scores)."""
    import torch
    w = bench.WORKLOADS[name]
    say(f"case: full-size {name} {w}")
    inp = bench.make_inputs(w, torch.device("cuda"))
    out = torch.empty(w["B"], dtype=torch.float32, device="cuda")
    for _, fn in bench.launches(ms(), w, inp, out):
        fn()
    torch.cuda.synchronize()
    return w, inp, out.cpu().numpy().astype(np.float64)


def release(inp):
    import torch
    inp.clear()
    torch.cuda.empty_cache()


def fixed_oracle(w, ids):
    """Oracle scores of the listed documents of a fixed-layout workload (regenerated)."""
    pool = w.get("pool") or w["B"]
    src = np.array([int(b) % pool for b in ids])
    Q = (gen.tokens(w["seed"], gen.S_QUERY, 0, w["q_len"], w["d"], w["dtype"]))
    if w["dtype"] == "i8":
        Dq, Ds = gen.fixed_docs_subset(w["seed"], src, w["nd"], w["d"], "i8")
        return oracle.maxsim_i8(Q[0], Q[1], Dq, Ds)[0]
    D = gen.fixed_docs_subset(w["seed"], src, w["nd"], w["d"], w["dtype"])
    return oracle.maxsim_fixed(Q, D, w["dtype"])


def test_headline_colbert_b100k_every_document():
    w, inp, got = run("colbert-b100k")
    release(inp)
    c = gen.fixed_corpus(w["seed"], w["B"], w["q_len"], w["nd"], w["d"], w["dtype"])
    want = oracle.maxsim_fixed(c.Q, c.D, w["dtype"])
    compare(got, want, what="colbert-b100k (all 100000 docs)")
    topk_agree(got, want, 100)


def _sampled(name, n=600, seed=0):
    w, inp, got = run(name)
    release(inp)
    rng = np.random.default_rng(seed)
    ids = np.unique(np.concatenate([[0, w["B"] - 1], rng.integers(0, w["B"], size=n)]))
    compare(got[ids], fixed_oracle(w, ids), what=f"{name} ({len(ids)} sampled docs)")
    pool = w.get("pool")
    if pool and pool < w["B"]:
        b = np.arange(w["B"])
        assert np.array_equal(got, got[b % pool]), "replicated documents must score identically"
    return got


@pytest.mark.parametrize("name", ["colbert-b1k", "colbert-b10k", "colbert-b500k", "colbert-nd32",
                                  "colbert-nd64", "colbert-nd256", "colbert-nd512", "colbert-fp16",
                                  "colbert-fp32", "dtile-d64", "dtile-d256", "dtile-d768"])
def test_fixed_workloads_sampled(name):
    _sampled(name)


@pytest.mark.parametrize("name", ["colpali-bf16-b175k", "colpali-i8-b175k"])
def test_colpali_scale_sampled(name):
    w, inp, got = run(name)
    release(inp)
    rng = np.random.default_rng(1)
    ids = np.unique(np.concatenate([[0, w["B"] - 1], rng.integers(0, w["B"], size=40)]))
    compare(got[ids], fixed_oracle(w, ids), what=f"{name} ({len(ids)} sampled docs)")
    b = np.arange(w["B"])
    assert np.array_equal(got, got[b % w["pool"]])


def test_csr_bf16_every_document():
    w, inp, got = run("csr-bf16")
    release(inp)
    c = gen.csr_corpus(w["seed"], w["B"], w["q_len"], w["d"], w["dtype"])
    compare(got, oracle.maxsim_csr(c.Q, c.D, c.offsets, w["dtype"]), what="csr-bf16 (all docs)")


@pytest.mark.parametrize("name", ["csr-pq", "fixed-pq"])
def test_pq_every_document(name):
    w, inp, got = run(name)
    release(inp)
    Q = gen.tokens(w["seed"], gen.S_QUERY, 0, w["q_len"], w["d"], w["dtype"])
    C = gen.codebook(w["seed"], bench.PQ_M, bench.PQ_K, bench.PQ_DSUB)
    T = oracle.pq_tables(Q, w["dtype"], C)
    if w["layout"] == "csr":
        off = gen.csr_offsets(gen.lengths(w["seed"], w["B"]))
        codes = gen.codes(w["seed"], int(off[-1]), bench.PQ_M, bench.PQ_K)
        want = oracle.maxsim_pq(T, codes, offsets=off)
    else:
        codes = gen.codes(w["seed"], w["B"] * w["nd"], bench.PQ_M, bench.PQ_K)
        want = oracle.maxsim_pq(T, codes, nd=w["nd"])
    compare(got, want, tol=PQ_TOL, what=f"{name} (all docs)")
