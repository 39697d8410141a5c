"""Pins of the MaxSim oracle: checks against things other than the oracle itself.

Each pin takes an `oracle.Oracle` and raises AssertionError on a mismatch. They are
run against the real oracle (test_oracle_pins.py) and against deliberately broken
copies of it (test_oracle_mutants.py), where at least one pin must fail.

Kinds of pin used:
  - hand-worked examples (tests/golden/hand_examples.json);
  - brute force on tiny inputs: numpy float64 that materialises the similarity tensor
    S[b, i, j] and reduces it (the naive method the pages contrast with), with numpy's
    own bf16 / fp16 decoding;
  - closed forms: one document token (score = <sum_i q_i, d_0>), one query token
    (max of a matrix-vector product), one-hot tokens (score = count of shared basis
    indices), doc == query with exactly unit-norm dyadic tokens (score = q_len);
  - invariants: permutation of document tokens, padding and neighbour independence,
    scaling by powers of two;
  - the planted near-duplicates of the 1000-document workload are the top-10;
  - gradients: Euler's identity for homogeneous functions (<dQ, Q> = <dD, D> = the
    weighted score), exact central differences on dyadic inputs, and the one-token
    closed form; argmax against the materialised tensor with exact ties.
"""
from __future__ import annotations

import json
import os

import numpy as np

import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


# ---- numpy decoding of stored values (independent of the oracle's C decoders) ----

def dec(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "fp16":
        return a.view(np.float16).astype(np.float64)
    return a.astype(np.float64)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round doubles to a storage format (via fp32, RNE) using numpy / the generator."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return gen.round_bf16(x32)
    if dtype == "fp16":
        return x32.astype(np.float16)
    return x32


def brute_dense(qd: np.ndarray, docs: list[np.ndarray]) -> np.ndarray:
    """Materialise S = Q . D_b^T per doc, max over doc tokens, sum over query tokens."""
    out = np.empty(len(docs))
    for b, Db in enumerate(docs):
        if Db.shape[0] == 0:
            out[b] = -np.inf
            continue
        S = np.einsum("ik,jk->ij", qd, Db)
        out[b] = S.max(axis=1).sum()
    return out


def _unit_rows(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


# ---------------------------------------------------------------- golden

def pin_golden_dense(orc):
    ex = json.load(open(GOLDEN))
    for e in ex["dense"]:
        Q = np.array(e["Q"], dtype=np.float32)
        lens = [len(doc) for doc in e["docs"]]
        nd = max(lens)
        d = Q.shape[1]
        D = np.full((len(lens), nd, d), 1e6, dtype=np.float32)  # padding garbage
        for b, doc in enumerate(e["docs"]):
            D[b, :len(doc)] = np.array(doc, dtype=np.float32)
        got = orc.maxsim_fixed(Q, D, "fp32", doc_lens=np.array(lens, np.int32))
        assert np.array_equal(got, np.array(e["expected"])), (e["name"], got)
        Dc = np.concatenate([np.array(doc, dtype=np.float32) for doc in e["docs"]])
        got = orc.maxsim_csr(Q, Dc, gen.csr_offsets(np.array(lens)), "fp32")
        assert np.array_equal(got, np.array(e["expected"])), (e["name"], "csr", got)


def pin_golden_int8(orc):
    ex = json.load(open(GOLDEN))
    for e in ex["int8"]:
        Q = np.array(e["Q"], dtype=np.int8)
        D = np.array(e["docs"], dtype=np.int8)
        s, tm, ta = orc.maxsim_i8(Q, np.array(e["q_scale"], np.float32), D,
                                  np.array(e["d_scale"], np.float32))
        assert np.array_equal(s, np.array(e["expected"])), (e["name"], s)
        assert np.array_equal(tm, np.array(e["tok_max"], np.float32)), (e["name"], tm)
        assert np.array_equal(ta, np.array(e["tok_arg"], np.int32)), (e["name"], ta)


def pin_golden_pq(orc):
    ex = json.load(open(GOLDEN))
    for e in ex["pq"]:
        Q = np.array(e["Q"], dtype=np.float32)
        C = np.array(e["C"], dtype=np.float32)
        T = orc.pq_tables(Q, "fp32", C)
        assert np.array_equal(T, np.array(e["tables"], np.float64)), (e["name"], T)
        codes = np.array(e["codes"], dtype=np.uint8)
        nd = codes.shape[1]
        got = orc.maxsim_pq(T, codes.reshape(-1, C.shape[0]), nd=nd)
        assert np.array_equal(got, np.array(e["expected"])), (e["name"], got)


# ---------------------------------------------------------------- brute force

def pin_brute_dense(orc):
    rng = np.random.default_rng(11)
    for dtype in ("bf16", "fp16", "fp32"):
        for d in (8, 64, 128):
            q_len, nd, B = int(rng.integers(1, 9)), int(rng.integers(1, 17)), 24
            Q = store(_unit_rows(rng, q_len, d), dtype)
            D = store(_unit_rows(rng, B * nd, d), dtype).reshape(B, nd, d)
            qd, Dd = dec(Q, dtype), dec(D, dtype)
            want = brute_dense(qd, list(Dd))
            got = orc.maxsim_fixed(Q, D, dtype)
            assert np.allclose(got, want, rtol=0, atol=1e-12), (dtype, d, np.abs(got - want).max())
            # masked: doc_lens in [0, nd]; masked rows hold large garbage
            lens = rng.integers(0, nd + 1, size=B).astype(np.int32)
            Dg = D.copy()
            for b in range(B):
                Dg[b, lens[b]:] = store(np.full((nd - lens[b], d), 60.0), dtype)
            want = brute_dense(qd, [Dd[b, :lens[b]] for b in range(B)])
            got = orc.maxsim_fixed(Q, Dg, dtype, doc_lens=lens)
            fin = np.isfinite(want)
            assert np.array_equal(np.isfinite(got), fin)
            assert np.all(got[~fin] == -np.inf)
            assert np.allclose(got[fin], want[fin], rtol=0, atol=1e-12), (dtype, d, "masked")
            # CSR with the same per-doc token counts
            lens = rng.integers(0, 20, size=B)
            off = gen.csr_offsets(lens)
            Dc = store(_unit_rows(rng, int(off[-1]), d), dtype)
            Dcd = dec(Dc, dtype)
            want = brute_dense(qd, [Dcd[off[b]:off[b + 1]] for b in range(B)])
            got = orc.maxsim_csr(Q, Dc, off, dtype)
            fin = np.isfinite(want)
            assert np.array_equal(np.isfinite(got), fin)
            assert np.allclose(got[fin], want[fin], rtol=0, atol=1e-12), (dtype, d, "csr")


def pin_brute_fp16_subnormal(orc):
    """Documents made only of fp16 subnormals: the score is carried by them alone."""
    rng = np.random.default_rng(12)
    q_len, nd, B, d = 4, 8, 6, 64
    Q = store(_unit_rows(rng, q_len, d), "fp16")
    raw = rng.integers(-1023, 1024, size=(B, nd, d))  # subnormal mantissas, +-man * 2^-24
    D = (np.sign(raw) * np.abs(raw) * 2.0 ** -24).astype(np.float16)
    assert np.all(np.abs(D.astype(np.float64)) < 2.0 ** -14)
    want = brute_dense(dec(Q, "fp16"), list(dec(D, "fp16")))
    got = orc.maxsim_fixed(Q, D, "fp16")
    assert np.allclose(got, want, rtol=1e-12, atol=0), np.abs(got - want).max()
    assert np.all(np.abs(want) > 0)


def pin_brute_int8(orc):
    rng = np.random.default_rng(13)
    for d in (16, 64, 128):
        q_len, nd, B = 5, 9, 20
        Q = rng.integers(-127, 128, size=(q_len, d)).astype(np.int8)
        D = rng.integers(-127, 128, size=(B, nd, d)).astype(np.int8)
        D[:, 4] = D[:, 1]  # exact duplicates -> argmax ties
        qs = (rng.random(q_len) * 0.02 + 1e-3).astype(np.float32)
        ds = (rng.random((B, nd)) * 0.02 + 1e-3).astype(np.float32)
        ds[:, 4] = ds[:, 1]
        s, tm, ta = orc.maxsim_i8(Q, qs, D, ds)
        dot = np.einsum("ik,bjk->bij", Q.astype(np.int64), D.astype(np.int64))
        v = dot.astype(np.float32) * (qs[None, :, None] * ds[:, None, :]).astype(np.float32)
        assert v.dtype == np.float32
        want_max = v.max(axis=2)
        want_arg = v.argmax(axis=2).astype(np.int32)  # first occurrence = lowest j
        assert np.array_equal(tm, want_max)
        assert np.array_equal(ta, want_arg)
        assert np.allclose(s, want_max.astype(np.float64).sum(axis=1), rtol=0, atol=1e-9)
        # literal int32 maxima: all scales 1
        s1, tm1, ta1 = orc.maxsim_i8(Q, np.ones(q_len, np.float32), D, np.ones((B, nd), np.float32))
        assert np.array_equal(tm1, dot.max(axis=2).astype(np.float32))
        assert np.array_equal(ta1, dot.argmax(axis=2).astype(np.int32))
        # CSR layout gives the same as the fixed layout
        off = gen.csr_offsets(np.full(B, nd))
        sc, tmc, tac = orc.maxsim_i8(Q, qs, D.reshape(-1, d), ds.reshape(-1), offsets=off)
        assert np.array_equal(sc, s) and np.array_equal(tmc, tm) and np.array_equal(tac, ta)


def pin_brute_pq(orc):
    """PQ scores equal brute-force MaxSim on the decoded vectors concat_m C[m, c_jm]."""
    rng = np.random.default_rng(14)
    for (M, K, dsub) in ((16, 256, 8), (4, 16, 2), (2, 8, 3)):
        d = M * dsub
        q_len, B = 7, 10
        C = rng.standard_normal((M, K, dsub)).astype(np.float32)
        Q = store(_unit_rows(rng, q_len, d), "bf16")
        qd = dec(Q, "bf16")
        T = orc.pq_tables(Q, "bf16", C)
        # tables: per-subspace matrix products
        for m in range(M):
            Tm = qd[:, m * dsub:(m + 1) * dsub] @ C[m].astype(np.float64).T
            assert np.allclose(T[:, m, :], Tm, rtol=0, atol=1e-12), ("tables", m)
        lens = rng.integers(1, 12, size=B)
        off = gen.csr_offsets(lens)
        codes = rng.integers(0, K, size=(int(off[-1]), M)).astype(np.uint8)
        recon = np.concatenate([C[m][codes[:, m]] for m in range(M)], axis=1).astype(np.float64)
        want = brute_dense(qd, [recon[off[b]:off[b + 1]] for b in range(B)])
        got = orc.maxsim_pq(T, codes, offsets=off)
        assert np.allclose(got, want, rtol=0, atol=1e-10), np.abs(got - want).max()


# ---------------------------------------------------------------- closed forms

def pin_dyadic_self(orc):
    """A document holding the query's exactly-unit-norm tokens scores exactly q_len."""
    rng = np.random.default_rng(15)
    for d in (64, 128, 256):
        q_len = 32
        Q = np.zeros((q_len, d))
        for i in range(q_len):
            idx = rng.permutation(d)[:64]
            Q[i, idx] = rng.choice([-0.125, 0.125], size=64)
        assert np.all(np.sum(Q * Q, axis=1) == 1.0)
        for dtype in ("bf16", "fp16", "fp32"):
            Qs = store(Q, dtype)
            others = store(_unit_rows(rng, 96, d), dtype)
            doc = np.concatenate([Qs[rng.permutation(q_len)], others])[None]
            got = orc.maxsim_fixed(Qs, doc, dtype)
            assert got[0] == float(q_len), (d, dtype, got)


def pin_one_token_doc(orc):
    """Nd = 1: score = <sum_i q_i, d_0>."""
    rng = np.random.default_rng(16)
    d = 128
    Q = store(_unit_rows(rng, 32, d), "bf16")
    D = store(_unit_rows(rng, 50, d), "bf16").reshape(50, 1, d)
    want = dec(D, "bf16")[:, 0, :] @ dec(Q, "bf16").sum(axis=0)
    got = orc.maxsim_fixed(Q, D, "bf16")
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def pin_one_query_token(orc):
    """q_len = 1: score = max over j of (D_b q)_j, a matrix-vector product and a max."""
    rng = np.random.default_rng(17)
    d = 64
    Q = store(_unit_rows(rng, 1, d), "fp32")
    D = store(_unit_rows(rng, 40 * 13, d), "fp32").reshape(40, 13, d)
    want = np.array([np.max(dec(D, "fp32")[b] @ dec(Q, "fp32")[0]) for b in range(40)])
    got = orc.maxsim_fixed(Q, D, "fp32")
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def pin_one_hot(orc):
    """One-hot tokens: each query basis vector scores 1 if present in the doc, else 0."""
    rng = np.random.default_rng(18)
    d = 64
    for _ in range(5):
        qa = rng.permutation(d)[:20]
        Q = np.zeros((20, d), np.float32)
        Q[np.arange(20), qa] = 1
        docs, want = [], []
        for b in range(12):
            db = rng.choice(d, size=int(rng.integers(1, 30)), replace=True)
            D = np.zeros((len(db), d), np.float32)
            D[np.arange(len(db)), db] = 1
            docs.append(D)
            want.append(len(set(qa.tolist()) & set(db.tolist())))
        off = gen.csr_offsets(np.array([len(x) for x in docs]))
        got = orc.maxsim_csr(store(Q, "bf16"), store(np.concatenate(docs), "bf16"), off, "bf16")
        assert np.array_equal(got, np.array(want, np.float64)), (got, want)


# ---------------------------------------------------------------- invariants

def pin_doc_permutation_and_duplicates(orc):
    rng = np.random.default_rng(19)
    d, nd = 128, 32
    Q = store(_unit_rows(rng, 32, d), "bf16")
    D = store(_unit_rows(rng, 8 * nd, d), "bf16").reshape(8, nd, d)
    base = orc.maxsim_fixed(Q, D, "bf16")
    P = D[:, rng.permutation(nd)]
    assert np.array_equal(orc.maxsim_fixed(Q, P, "bf16"), base)
    dup = np.concatenate([D, D[:, :5]], axis=1)
    assert np.array_equal(orc.maxsim_fixed(Q, dup, "bf16"), base)


def pin_padding_and_neighbours(orc):
    """Masked padding and neighbouring CSR documents never change a score."""
    rng = np.random.default_rng(20)
    d = 64
    Q = store(_unit_rows(rng, 16, d), "bf16")
    lens = np.array([5, 17, 1, 9, 30])
    docs = [store(_unit_rows(rng, L, d), "bf16") for L in lens]
    alone = np.array([orc.maxsim_csr(Q, x, np.array([0, len(x)]), "bf16")[0] for x in docs])
    huge = store(np.full((3, d), 100.0), "bf16")
    parts, off = [], [0]
    for x in docs:
        parts += [x, huge]
        off.append(off[-1] + len(x))
        off.append(off[-1] + 3)
    Dc = np.concatenate(parts)
    got = orc.maxsim_csr(Q, Dc, np.array(off), "bf16")[0::2]
    assert np.array_equal(got, alone)
    nd = 40
    Df = np.empty((len(lens), nd, d), np.uint16)
    Df[...] = store(np.full(d, -100.0), "bf16")
    for b, x in enumerate(docs):
        Df[b, :len(x)] = x
    got = orc.maxsim_fixed(Q, Df, "bf16", doc_lens=lens.astype(np.int32))
    assert np.array_equal(got, alone)


def pin_power_of_two_scaling(orc):
    rng = np.random.default_rng(21)
    d = 128
    Q = _unit_rows(rng, 32, d).astype(np.float32)
    D = _unit_rows(rng, 10 * 20, d).astype(np.float32).reshape(10, 20, d)
    base = orc.maxsim_fixed(Q, D, "fp32")
    for k in (-3, 1, 4):
        got = orc.maxsim_fixed((Q * 2.0 ** k).astype(np.float32), D, "fp32")
        assert np.array_equal(got, base * 2.0 ** k), k


def pin_query_permutation(orc):
    rng = np.random.default_rng(22)
    d = 128
    Q = store(_unit_rows(rng, 32, d), "fp16")
    D = store(_unit_rows(rng, 6 * 40, d), "fp16").reshape(6, 40, d)
    base = orc.maxsim_fixed(Q, D, "fp16")
    got = orc.maxsim_fixed(Q[rng.permutation(32)], D, "fp16")
    assert np.allclose(got, base, rtol=0, atol=1e-12)
    # a zero query token adds exactly 0 (its max over a non-empty doc is 0)
    Qz = np.concatenate([Q, np.zeros((1, d), np.float16)])
    assert np.array_equal(orc.maxsim_fixed(Qz, D, "fp16"), base)


def pin_planted_top10(orc):
    """1000 docs of 128 tokens, 10 planted near-duplicates of the query: they are the top-10."""
    c = gen.fixed_corpus(gen.SEEDS["C1"], 1000, 32, 128, 128, "bf16", n_plant=10)
    s = orc.maxsim_fixed(c.Q, c.D, "bf16")
    top = np.argsort(-s, kind="stable")[:10]
    assert set(top.tolist()) == set(c.planted.tolist()), (top, c.planted)
    others = np.delete(s, c.planted)
    assert s[c.planted].min() > 20.0 and others.max() < 12.0, (s[c.planted].min(), others.max())


# ---------------------------------------------------------------- argmax and gradients

def brute_argmax(qd: np.ndarray, docs: list[np.ndarray]):
    """Per-token maxima and argmax from the materialised S (numpy's argmax returns the
    first maximum, i.e. the lowest document index)."""
    q_len = qd.shape[0]
    tm = np.full((len(docs), q_len), -np.inf)
    ta = np.full((len(docs), q_len), -1, dtype=np.int64)
    for b, Db in enumerate(docs):
        if Db.shape[0]:
            S = np.einsum("ik,jk->ij", qd, Db)
            tm[b], ta[b] = S.max(axis=1), S.argmax(axis=1)
    return tm, ta


def pin_argmax_brute(orc):
    """Per-token maxima and argmax against the materialised similarity tensor, with exact
    ties (duplicated document tokens: the lower index wins) and empty CSR documents."""
    rng = np.random.default_rng(21)
    for dtype in ("bf16", "fp16", "fp32"):
        q_len, nd, d, B = 7, 9, 64, 12
        Q = store(_unit_rows(rng, q_len, d), dtype)
        D = store(_unit_rows(rng, B * nd, d), dtype).reshape(B, nd, d)
        D[3, 6] = D[3, 2]          # a tie: token 2 must win over its copy at 6
        D[5, 1:] = D[5, 0]         # all tokens equal: every argmax is 0
        qd, Dd = dec(Q, dtype), dec(D, dtype)
        s, tm, ta = orc.maxsim_argmax(Q, D, dtype)
        wtm, wta = brute_argmax(qd, list(Dd))
        assert np.array_equal(ta, wta), (dtype, "fixed argmax")
        assert np.allclose(tm, wtm, rtol=0, atol=1e-12)
        assert np.allclose(s, wtm.sum(axis=1), rtol=0, atol=1e-12)
        assert np.all(ta[5] == 0)
        lens = np.array([0, 1, 5, 0, 17, 3, 9, 2])
        off = gen.csr_offsets(lens)
        Dc = store(_unit_rows(rng, int(off[-1]), d), dtype)
        Dc[off[4] + 11] = Dc[off[4] + 4]
        docs = [dec(Dc, dtype)[off[b]:off[b + 1]] for b in range(len(lens))]
        s, tm, ta = orc.maxsim_argmax(Q, Dc, dtype, offsets=off)
        wtm, wta = brute_argmax(qd, docs)
        assert np.array_equal(ta, wta), (dtype, "csr argmax")
        assert np.all(ta[lens == 0] == -1) and np.all(np.isneginf(tm[lens == 0]))
        fin = lens > 0
        assert np.allclose(tm[fin], wtm[fin], rtol=0, atol=1e-12)
        assert np.all(np.isneginf(s[~fin]))


def _grad_case(rng, dtype, offsets_mode):
    q_len, d = 6, 64
    Q = store(_unit_rows(rng, q_len, d), dtype)
    if offsets_mode:
        lens = np.array([3, 0, 11, 1, 7, 16, 5])
        off = gen.csr_offsets(lens)
        D = store(_unit_rows(rng, int(off[-1]), d), dtype)
        n_docs = len(lens)
    else:
        off, n_docs = None, 9
        D = store(_unit_rows(rng, n_docs * 8, d), dtype).reshape(n_docs, 8, d)
    g = rng.standard_normal(n_docs).astype(np.float32)
    return Q, D, off, g


def pin_backward_euler(orc):
    """The score is positively homogeneous of degree one in Q and, separately, in D, so
    by Euler's theorem <dQ, Q> = <dD, D> = sum_b g_b score_b (empty documents excluded).
    A wrong row, a dropped factor or a wrong sign in either gradient breaks it."""
    rng = np.random.default_rng(22)
    for dtype in ("bf16", "fp16", "fp32"):
        for csr in (False, True):
            Q, D, off, g = _grad_case(rng, dtype, csr)
            s, _, ta = orc.maxsim_argmax(Q, D, dtype, offsets=off)
            dQ, dD = orc.maxsim_backward(Q, D, dtype, ta, g, offsets=off)
            fin = np.isfinite(s)
            want = float(np.sum(g[fin].astype(np.float64) * s[fin]))
            eq = float(np.sum(dQ * dec(Q, dtype)))
            ed = float(np.sum(dD * dec(D, dtype)))
            assert abs(eq - want) <= 1e-9 * (1 + abs(want)), (dtype, csr, eq, want)
            assert abs(ed - want) <= 1e-9 * (1 + abs(want)), (dtype, csr, ed, want)
            assert dD.shape == D.shape and dQ.shape == Q.shape


def pin_backward_finite_difference(orc):
    """Central differences of L = sum_b g_b score_b on dyadic fp32 inputs whose argmax is
    unique by a margin: L is linear in Q (and in D) near the point, every value is exact
    in double, so (L(x + eV) - L(x - eV)) / 2e equals <grad, V> exactly."""
    rng = np.random.default_rng(23)
    q_len, nd, d, B = 5, 6, 8, 7
    for _ in range(100):
        Q = (rng.integers(-8, 9, size=(q_len, d)) / 8.0).astype(np.float32)
        D = (rng.integers(-8, 9, size=(B, nd, d)) / 8.0).astype(np.float32)
        S = np.einsum("ik,bjk->bij", Q.astype(np.float64), D.astype(np.float64))
        top2 = np.sort(S, axis=2)[:, :, -2:]
        if np.all(top2[:, :, 1] - top2[:, :, 0] >= 1.0 / 64):
            break
    else:
        raise AssertionError("no input with a unique argmax margin")
    g = (rng.integers(-4, 5, size=B) / 4.0).astype(np.float32)
    _, _, ta = orc.maxsim_argmax(Q, D, "fp32")
    dQ, dD = orc.maxsim_backward(Q, D, "fp32", ta, g)
    eps = 2.0 ** -12

    def L(Qx, Dx):
        return float(np.sum(g.astype(np.float64) * orc.maxsim_fixed(Qx, Dx, "fp32")))

    for _ in range(4):
        V = rng.integers(-1, 2, size=Q.shape).astype(np.float32)
        fd = (L(Q + eps * V, D) - L(Q - eps * V, D)) / (2 * eps)
        assert fd == float(np.sum(dQ * V)), ("dQ", fd, float(np.sum(dQ * V)))
        W = rng.integers(-1, 2, size=D.shape).astype(np.float32)
        fd = (L(Q, D + eps * W) - L(Q, D - eps * W)) / (2 * eps)
        assert fd == float(np.sum(dD * W)), ("dD", fd, float(np.sum(dD * W)))


def pin_backward_one_token_docs(orc):
    """Documents of one token: every query token picks it, so dD[b, 0] = g_b sum_i q_i
    and dQ[i] = sum_b g_b d_b (closed form, for every i)."""
    rng = np.random.default_rng(24)
    Q = store(_unit_rows(rng, 5, 64), "bf16")
    D = store(_unit_rows(rng, 9, 64), "bf16").reshape(9, 1, 64)
    g = rng.standard_normal(9).astype(np.float32)
    _, _, ta = orc.maxsim_argmax(Q, D, "bf16")
    assert np.all(ta == 0)
    dQ, dD = orc.maxsim_backward(Q, D, "bf16", ta, g)
    qd, Dd = dec(Q, "bf16"), dec(D, "bf16")[:, 0]
    assert np.allclose(dD[:, 0], np.outer(g, qd.sum(axis=0)), rtol=0, atol=1e-12)
    assert np.allclose(dQ, np.broadcast_to(g.astype(np.float64) @ Dd, dQ.shape), rtol=0, atol=1e-12)


def pin_topk_brute(orc):
    """Top-k against repeated extraction of the best remaining entry (largest score, lowest
    index among equals) on small rows with ties and -inf."""
    import oracle as oracle_module
    rng = np.random.default_rng(25)
    for n, k in ((1, 1), (7, 3), (20, 20), (25, 30), (64, 10)):
        S = (rng.integers(-4, 5, size=(3, n)) / 4.0).astype(np.float32)
        S[:, ::5] = -np.inf
        vals, idx = oracle_module.topk(S, k)
        for r in range(3):
            left = list(range(n))
            for j in range(k):
                if not left:
                    assert idx[r, j] == -1 and vals[r, j] == -np.inf
                    continue
                best = left[0]
                for i in left:
                    if S[r, i] > S[r, best]:
                        best = i
                left.remove(best)
                assert idx[r, j] == best and vals[r, j] == S[r, best], (n, k, r, j)


PINS = [
    pin_golden_dense, pin_golden_int8, pin_golden_pq,
    pin_brute_dense, pin_brute_fp16_subnormal, pin_brute_int8, pin_brute_pq,
    pin_dyadic_self, pin_one_token_doc, pin_one_query_token, pin_one_hot,
    pin_doc_permutation_and_duplicates, pin_padding_and_neighbours, pin_power_of_two_scaling,
    pin_query_permutation, pin_planted_top10,
    pin_argmax_brute, pin_backward_euler, pin_backward_finite_difference,
    pin_backward_one_token_docs, pin_topk_brute,
]
