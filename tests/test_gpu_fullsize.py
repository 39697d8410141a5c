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
    out = torch.empty(w.get("n_q", 1) * w["B"], dtype=torch.float32, device="cuda")
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
                                  "colbert-fp32", "dtile-d64", "dtile-d256", "dtile-d768",
                                  "colbert-i8-b100k"])
def test_fixed_workloads_sampled(name):
    _sampled(name)


@pytest.mark.parametrize("name", ["colpali-bf16-b1k", "colpali-bf16-b10k", "colpali-bf16-b50k",
                                  "colpali-bf16-b175k", "colpali-i8-b1k", "colpali-i8-b10k",
                                  "colpali-i8-b50k", "colpali-i8-b175k"])
def test_colpali_scale_sampled(name):
    w, inp, got = run(name)
    release(inp)
    rng = np.random.default_rng(1)
    ids = np.unique(np.concatenate([[0, w["B"] - 1], rng.integers(0, w["B"], size=40)]))
    compare(got[ids], fixed_oracle(w, ids), what=f"{name} ({len(ids)} sampled docs)")
    if w.get("pool"):  # corpora built from a pool: every replica equals its pool document
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
        # the bench's codes: nearest-centroid codes of the generated tokens
        codes = bench.pq_codes(w["seed"], int(off[-1]), C)
        want = oracle.maxsim_pq(T, codes, offsets=off)
    else:
        codes = bench.pq_codes(w["seed"], w["B"] * w["nd"], C)
        want = oracle.maxsim_pq(T, codes, nd=w["nd"])
    compare(got, want, tol=PQ_TOL, what=f"{name} (all docs)")


def _argmax_rule(Q, docs_of_ids, ids, ta_gpu, ta_orc, tm_orc, margin):
    """Where the GPU argmax differs from the oracle's, the GPU's token must be within
    `margin` of the maximum (a near-tie that fp32 rounding may decide either way)."""
    diff = np.argwhere(ta_gpu[ids] != ta_orc[ids])
    for k, i in diff:
        b = ids[k]
        row = docs_of_ids(b)[ta_gpu[b, i]]
        assert float(row @ Q[i]) >= tm_orc[b, i] - margin, (b, i, ta_gpu[b, i], ta_orc[b, i])
    return len(diff)


@pytest.mark.parametrize("name", ["train-colbert-b100k", "train-csr"])
def test_train_step_full_size(name):
    """The training step at the headline shape: forward scores, per-token maxima and argmax
    on every document; then the backward, given the oracle's argmax in the same launch
    configuration: dQ element by element, dD on sampled documents."""
    import torch

    from oracle_pins import dec
    from test_gpu_backward import check_bound
    w, inp, got = run(name)
    ta_gpu = inp["tok_arg"].cpu().numpy()
    tm_gpu = inp["tok_max"].cpu().numpy().astype(np.float64)
    if w["layout"] == "fixed":
        c = gen.fixed_corpus(w["seed"], w["B"], w["q_len"], w["nd"], w["d"], w["dtype"])
        Dd = lambda b: dec(c.D[b], w["dtype"])
    else:
        c = gen.csr_corpus(w["seed"], w["B"], w["q_len"], w["d"], w["dtype"])
        Dd = lambda b: dec(c.D[c.offsets[b]:c.offsets[b + 1]], w["dtype"])
    ws, tm, ta = oracle.maxsim_argmax(c.Q, c.D, w["dtype"], offsets=c.offsets)
    compare(got, ws, what=f"{name} scores (all docs)")
    assert np.abs(tm_gpu - tm).max() <= 2e-5
    Qd = dec(c.Q, w["dtype"])
    nd = _argmax_rule(Qd, Dd, np.arange(w["B"]), ta_gpu, ta, tm, 2e-5)
    say(f"  {name}: argmax differs from the oracle's on {nd} of {ta.size} near-tied pairs")

    # backward from the oracle's argmax, same entry point and buffers as the step
    g = inp["grad"].cpu().numpy()
    inp["tok_arg"].copy_(torch.from_numpy(ta))
    ms().maxsim_backward(inp["Q"], inp["D"], inp["tok_arg"], inp["grad"], inp["offsets"],
                         grad_dtype=inp["D"].dtype, dQ=inp["dQ"], dD=inp["dD"],
                         workspace=inp["workspace"])
    torch.cuda.synchronize()
    gQ = inp["dQ"].float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(7)
    ids = np.unique(np.concatenate([[0, w["B"] - 1], rng.integers(0, w["B"], size=400)]))
    if w["layout"] == "fixed":
        gD = inp["dD"][torch.from_numpy(ids).cuda()].float().cpu().numpy().astype(np.float64)
    else:
        rows = np.concatenate([np.arange(c.offsets[b], c.offsets[b + 1]) for b in ids])
        gD = inp["dD"][torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    n_ranges = ms().backward_workspace_size(w["q_len"], w["d"], w["B"]) // (w["q_len"] * w["d"] * 4)
    release(inp)

    absQ, absD = c.Q & 0x7fff, c.D & 0x7fff  # bf16 |x|: clear the sign bit
    dQ, _ = oracle.maxsim_backward(c.Q, c.D, w["dtype"], ta, g, offsets=c.offsets, want_dD=False)
    mQ, _ = oracle.maxsim_backward(absQ, absD, w["dtype"], ta, np.abs(g), offsets=c.offsets,
                                   want_dD=False)
    per_range = -(-w["B"] // n_ranges)
    check_bound(gQ, dQ, mQ, per_range, w["dtype"], f"{name} dQ")
    # dD rows of the sampled documents depend only on those documents
    if w["layout"] == "fixed":
        sub, soff = c.D[ids], None
    else:
        lens = c.offsets[ids + 1] - c.offsets[ids]
        soff = gen.csr_offsets(lens)
        sub = c.D[rows]
    dD = oracle.maxsim_backward(c.Q, sub, w["dtype"], ta[ids], g[ids], offsets=soff)[1]
    mD = oracle.maxsim_backward(absQ, sub & 0x7fff, w["dtype"], ta[ids], np.abs(g[ids]),
                                offsets=soff)[1]
    check_bound(gD, dD, mD, w["q_len"], w["dtype"], f"{name} dD ({len(ids)} sampled docs)")


@pytest.mark.parametrize("name", ["batch-colbert-q32-b100k", "batch-colbert-q8-b100k"])
def test_batch_colbert_sampled(name):
    """32 (8) queries against the 100K-document ColBERT corpus in the bench's launch: every
    query's scores on sampled documents against the oracle."""
    w, inp, got = run(name)
    release(inp)
    got = got.reshape(w["n_q"], w["B"])
    rng = np.random.default_rng(3)
    ids = np.unique(np.concatenate([[0, w["B"] - 1], rng.integers(0, w["B"], size=150)]))
    Q = gen.tokens(w["seed"], gen.S_QUERY, 0, w["n_q"] * w["q_len"], w["d"], w["dtype"])
    D = gen.fixed_docs_subset(w["seed"], ids, w["nd"], w["d"], w["dtype"])
    want = oracle.maxsim_batch(Q.reshape(w["n_q"], w["q_len"], w["d"]), D, w["dtype"])
    compare(got[:, ids].ravel(), want.ravel(),
            what=f"{name} ({len(ids)} sampled docs x {w['n_q']} queries)")


def test_batch_q32_topk100():
    """32 queries, then the top-100 of each query's row, in the bench's launch: the selection
    is exact on the GPU's scores (values bit for bit, indices equal) for every query."""
    w, inp, got = run("batch-colbert-q32-topk100-b100k")
    idx = inp["topk_idx"].cpu().numpy().astype(np.int64)
    vals = inp["topk_vals"].cpu().numpy()
    release(inp)
    g32 = got.astype(np.float32).reshape(w["n_q"], w["B"])
    wv, wi = oracle.topk(g32, 100)
    assert np.array_equal(idx.reshape(wi.shape), wi)
    assert np.array_equal(vals.reshape(wv.shape).view(np.uint32), wv.view(np.uint32))


def test_train_colpali_full_size():
    """The training step at the ColPali shape (Lq = Ld = 1024, d = 128, 10K documents from a
    pool of 2048) in the bench's launch. Forward: scores, per-token maxima and argmax of
    sampled documents against the oracle, and every replica equal to its pool document.
    Backward (from the step's own argmax, at full size): Euler's identity for a function
    positively homogeneous of degree one, <dQ, Q> = <dD, D> = sum_b g_b score_b, within
    the rounding of the bf16 gradients (2^-8 sum |dQ| |Q|) plus the score tolerance."""
    import torch

    from oracle_pins import dec
    w, inp, got = run("train-colpali-b10k")
    pool, B = w["pool"], w["B"]
    ta_gpu = inp["tok_arg"].cpu().numpy()
    tm_gpu = inp["tok_max"].cpu().numpy().astype(np.float64)
    b = np.arange(B)
    assert np.array_equal(got, got[b % pool]) and np.array_equal(ta_gpu, ta_gpu[b % pool])
    g = inp["grad"].cpu().numpy().astype(np.float64)

    def dot64(x, y):
        s = 0.0
        for r0 in range(0, x.shape[0], 1 << 20):
            s += float((x[r0:r0 + (1 << 20)].double() * y[r0:r0 + (1 << 20)].double()).sum())
        return s

    def absdot64(x, y):
        s = 0.0
        for r0 in range(0, x.shape[0], 1 << 20):
            s += float((x[r0:r0 + (1 << 20)].double().abs() *
                        y[r0:r0 + (1 << 20)].double().abs()).sum())
        return s

    Qt, Dt = inp["Q"], inp["D"]
    Df = Dt.reshape(B * w["nd"], w["d"])
    target = float(np.dot(g, got))
    tol = float(np.abs(g).sum()) * TOL

    def euler(dQ, dD, rel, what):
        dD = dD.reshape(B * w["nd"], w["d"])
        eq, eqb = dot64(dQ, Qt), rel * absdot64(dQ, Qt) + tol
        ed, edb = dot64(dD, Df), rel * absdot64(dD, Df) + tol
        say(f"  {what}: sum g score {target:.3f}; <dQ,Q> off by {abs(eq - target):.3e} "
            f"(bound {eqb:.3e}), <dD,D> off by {abs(ed - target):.3e} (bound {edb:.3e})")
        assert abs(eq - target) <= eqb and abs(ed - target) <= edb, what

    # the step's bf16 gradients: one rounding to bf16 (2^-8) per element dominates
    euler(inp["dQ"], inp["dD"], 2.0 ** -8, "bf16 gradients")
    # the same backward with fp32 gradients: dD rows sum at most q_len query rows and scale
    # by g once, dQ sums fp32 partials of a few documents per range in double:
    # gamma_{q_len + 2} covers both
    dQ32, dD32 = ms().maxsim_backward(Qt, Dt, inp["tok_arg"], inp["grad"], None,
                                      grad_dtype=torch.float32, workspace=inp["workspace"])
    torch.cuda.synchronize()
    n = w["q_len"] + 2
    euler(dQ32, dD32, n * 2.0 ** -24 / (1 - n * 2.0 ** -24), "fp32 gradients")
    del dQ32, dD32
    release(inp)

    ids = np.array([0, 1, pool - 1])
    Q = gen.tokens(w["seed"], gen.S_QUERY, 0, w["q_len"], w["d"], w["dtype"])
    D = gen.fixed_docs_subset(w["seed"], ids, w["nd"], w["d"], w["dtype"])
    ws, tm, ta = oracle.maxsim_argmax(Q, D, w["dtype"])
    compare(got[ids], ws, what="train-colpali scores (sampled docs)")
    assert np.abs(tm_gpu[ids] - tm).max() <= 2e-5
    Qd = dec(Q, w["dtype"])
    nd = _argmax_rule(Qd, lambda k: dec(D[k], w["dtype"]), np.arange(len(ids)), ta_gpu[ids], ta,
                      tm, 2e-5)
    say(f"  train-colpali: argmax differs from the oracle's on {nd} near-tied pairs")


def test_topk_after_headline_scoring():
    """Scoring + top-100 at the headline shape in the bench's launch: the selection is exact
    on the GPU's scores, and agrees with the oracle's ranking of its own scores except at
    ties within the tolerance."""
    w, inp, got = run("colbert-topk100-b100k")
    idx = inp["topk_idx"].cpu().numpy().astype(np.int64)
    vals = inp["topk_vals"].cpu().numpy()
    release(inp)
    g32 = got.astype(np.float32)
    wv, wi = oracle.topk(g32, 100)
    assert np.array_equal(idx, wi[0]) and np.array_equal(vals.view(np.uint32), wv[0].view(np.uint32))
    c = gen.fixed_corpus(w["seed"], w["B"], w["q_len"], w["nd"], w["d"], w["dtype"])
    topk_agree(got, oracle.maxsim_fixed(c.Q, c.D, w["dtype"]), 100)
