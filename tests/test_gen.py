"""The seeded input generator: determinism, distributions and storage rounding."""
import numpy as np
import torch

import gen


def test_same_seed_same_bytes_and_thread_independent():
    a = gen.tokens(7, gen.S_DOCS, 0, 3000, 128, "bf16", nthreads=1)
    b = gen.tokens(7, gen.S_DOCS, 0, 3000, 128, "bf16", nthreads=8)
    assert np.array_equal(a, b)
    c = gen.tokens(8, gen.S_DOCS, 0, 3000, 128, "bf16", nthreads=8)
    assert not np.array_equal(a, c)


def test_counter_based_rows():
    full = gen.tokens(3, gen.S_DOCS, 0, 40, 64, "fp32")
    part = gen.tokens(3, gen.S_DOCS, 17, 9, 64, "fp32")
    assert np.array_equal(full[17:26], part)


def test_unit_norm_after_rounding():
    x = gen.tokens(2, gen.S_DOCS, 0, 2000, 128, "bf16")
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    n = np.linalg.norm(xf, axis=1)
    assert np.all(np.abs(n - 1.0) < 4e-3)
    f = gen.tokens(2, gen.S_DOCS, 0, 2000, 128, "f64")
    assert np.allclose(np.linalg.norm(f, axis=1), 1.0, atol=1e-14)
    # Gaussian marginals: mean ~0, per-coordinate variance ~1/d
    assert abs(f.mean()) < 2e-3 and abs(f.var() * 128 - 1.0) < 0.02


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.round_bf16(x), want)


def test_fp16_rounding_matches_numpy_including_subnormals():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(20000) * 3e-6).astype(np.float32),   # subnormal
                        (rng.standard_normal(2000) * 1e5).astype(np.float32),     # overflow
                        np.array([65504.0, 65519.0, 65520.0, 2.0 ** -24, 2.0 ** -25,
                                  3 * 2.0 ** -26, 0.0, -0.0], np.float32)])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16)
    assert np.array_equal(gen.round_f16(x).view(np.uint16), want.view(np.uint16))


def test_storage_is_rounded_double():
    f = gen.tokens(5, gen.S_QUERY, 0, 32, 128, "f64")
    assert np.array_equal(gen.tokens(5, gen.S_QUERY, 0, 32, 128, "fp32"), f.astype(np.float32))
    assert np.array_equal(gen.tokens(5, gen.S_QUERY, 0, 32, 128, "fp16"),
                          f.astype(np.float32).astype(np.float16))
    assert np.array_equal(gen.tokens(5, gen.S_QUERY, 0, 32, 128, "bf16"),
                          gen.round_bf16(f.astype(np.float32)))


def test_int8_quantiser():
    f = gen.tokens(6, gen.S_DOCS, 0, 500, 128, "f64")
    q, s = gen.tokens(6, gen.S_DOCS, 0, 500, 128, "i8")
    assert np.array_equal(s, (np.abs(f).max(axis=1) / 127.0).astype(np.float32))
    assert np.all(np.abs(q.astype(np.int32)).max(axis=1) == 127)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    err = np.abs(q * s[:, None].astype(np.float64) - f)
    assert np.all(err <= s[:, None] * 0.5 + 1e-9)
    assert np.array_equal(q, np.clip(np.rint(f / s[:, None].astype(np.float64)), -127, 127))


def test_lognormal_lengths():
    L = gen.lengths(5, 100000)
    assert L.min() >= 8 and L.max() <= 512
    assert np.median(L) == 70
    assert 78 < L.mean() < 81
    assert np.array_equal(L, gen.lengths(5, 100000))


def test_planting_and_subset_regeneration():
    c = gen.fixed_corpus(1, 1000, 32, 128, 128, "bf16", n_plant=10)
    assert len(set(c.planted.tolist())) == 10
    plain = gen.fixed_corpus(1, 1000, 32, 128, 128, "bf16", n_plant=0)
    changed = np.nonzero(np.any(c.D != plain.D, axis=(1, 2)))[0]
    assert set(changed.tolist()) == set(c.planted.tolist())
    for b in c.planted:
        rows = np.nonzero(np.any(c.D[b] != plain.D[b], axis=1))[0]
        assert len(rows) == 32
    ids = [0, int(c.planted[0]), 999, int(c.planted[3])]
    sub = gen.fixed_docs_subset(1, ids, 128, 128, "bf16", n_plant_ids=c.planted, q_len=32)
    assert np.array_equal(sub, c.D[ids])


def test_csr_planting_short_docs():
    lens = np.array([8, 40, 12, 100, 20], np.int32)
    c = gen.csr_corpus(9, 5, 32, 64, "bf16", lens=lens, n_plant=3)
    plain = gen.csr_corpus(9, 5, 32, 64, "bf16", lens=lens, n_plant=0)
    for b in c.planted:
        s0, s1 = c.offsets[b], c.offsets[b + 1]
        changed = np.any(c.D[s0:s1] != plain.D[s0:s1], axis=1).sum()
        assert changed == min(32, lens[b])


def test_codes_and_codebook():
    C = gen.codebook(5)
    assert C.shape == (16, 256, 8)
    assert np.allclose(np.linalg.norm(C.astype(np.float64), axis=2), 1.0, atol=1e-6)
    cd = gen.codes(5, 10000)
    assert cd.shape == (10000, 16)
    counts = np.bincount(cd.ravel(), minlength=256)
    assert counts.min() > 400 and counts.max() < 860
    x = gen.tokens(5, gen.S_DOCS, 0, 50, 128, "f64")
    enc = gen.pq_encode(x, C)
    dist = ((x.reshape(50, 16, 1, 8) - C[None].astype(np.float64)) ** 2).sum(-1)
    assert np.array_equal(enc, dist.argmin(-1).astype(np.uint8))


def test_encoded_codes_equal_nearest_centroid_of_generated_tokens():
    """gen.encoded_codes (tokens generated and encoded in one threaded pass, centroid loop
    innermost) gives the codes pq_encode gives for the same generated tokens, for any
    thread count and row offset."""
    C = gen.codebook(5)
    x = gen.tokens(5, gen.S_DOCS, 100, 700, 128, "f64")
    want = gen.pq_encode(x, C)
    for nt in (1, 3, 8):
        assert np.array_equal(gen.encoded_codes(5, gen.S_DOCS, 100, 700, C, nthreads=nt), want)
    # with the ties-to-lowest rule, a token equal to a centroid's sub-vectors takes it
    assert np.array_equal(gen.pq_encode(np.repeat(C[:, 3, :].reshape(1, -1).astype(np.float64), 2, 0),
                                        C), np.full((2, 16), 3, np.uint8))
