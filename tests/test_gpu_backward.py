"""GPU parity of the forward with per-token maxima and argmax, and of the backward pass.

Argmax. Where floating point decides the index, the GPU (fp32 sums) and the oracle
(float64) may pick different tokens when two similarities are closer than the rounding
error. So: per-token maxima within MARGIN of the oracle's; the argmax equals the
oracle's wherever the oracle's best and second-best similarities differ by more than
2 * MARGIN, and elsewhere indexes a token whose oracle similarity is within MARGIN of
the maximum. Exact duplicates of a token have bit-identical fp32 similarities, so there
the lowest index is required. The scores equal the plain scoring entry point's bit for
bit (same arithmetic).

MARGIN: a bf16 / fp16 product is exact in fp32 and a unit-norm dot over d terms carries
at most gamma_d * sum|q_k d_k| <= d * 2^-24 of accumulation error (7.6e-6 at d = 128);
fp32 inputs add one rounding per product. 2e-5 covers d <= 256 with margin; d = 768
uses 6e-5.

Backward. The GPU backward is given the oracle's argmax (an oracle output may be a GPU
input) and compared with the oracle's gradients element by element within the fp32
summation bound gamma_{n+1} * M (n = number of terms, M = sum of |terms|, obtained by
running the oracle on |Q|, |D| and |g|: the gradients are linear in each), plus one
rounding to the gradient type (2^-8 relative for bf16, 2^-11 for fp16, plus 2^-25
absolute for fp16 subnormals).
"""
import numpy as np
import pytest

import gen
import oracle
from gpu_util import ms, say
from oracle_pins import dec

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24
# rounding of a gradient to its type: relative unit roundoff, and half the subnormal
# spacing (fp16 subnormals start below 6.1e-5; bf16 shares fp32's exponent range)
U_GRAD = {"fp32": 0.0, "bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
ETA_GRAD = {"fp32": 0.0, "bf16": 2.0 ** -134, "fp16": 2.0 ** -25}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ms()


def margin_for(d):
    return 2e-5 if d <= 256 else 6e-5


def dev(a, dtype):
    return gen.to_device(a, dtype)


def docs_of(c):
    """Decoded documents of a corpus as a list of [len, d] float64 arrays."""
    Dd = dec(c.D, c.dtype)
    if c.offsets is None:
        return list(Dd)
    return [Dd[c.offsets[b]:c.offsets[b + 1]] for b in range(len(c.offsets) - 1)]


def gpu_argmax(c):
    import torch
    Q, D = dev(c.Q, c.dtype), dev(c.D, c.dtype)
    off = None if c.offsets is None else torch.from_numpy(c.offsets).cuda()
    s, tm, ta = ms().maxsim_score_argmax(Q, D, off)
    plain = ms().maxsim_score_fixed(Q, D) if off is None else ms().maxsim_score(Q, D, off)
    torch.cuda.synchronize()
    return s.cpu().numpy(), tm.cpu().numpy(), ta.cpu().numpy(), plain.cpu().numpy()


def check_argmax(c, what):
    s, tm, ta, plain = gpu_argmax(c)
    assert np.array_equal(s.view(np.uint32), plain.view(np.uint32)), f"{what}: scores differ"
    ws, wtm, wta = oracle.maxsim_argmax(c.Q, c.D, c.dtype, offsets=c.offsets)
    qd = dec(c.Q, c.dtype)
    mg = margin_for(c.d)
    unique = forced = 0
    for b, Db in enumerate(docs_of(c)):
        if Db.shape[0] == 0:
            assert np.all(ta[b] == -1) and np.all(np.isneginf(tm[b])), f"{what}: empty doc {b}"
            continue
        S = qd @ Db.T
        top2 = np.sort(S, axis=1)[:, -2:] if Db.shape[0] > 1 else np.hstack([S - 1, S])
        assert np.all(np.abs(tm[b] - wtm[b]) <= mg), (what, b, np.abs(tm[b] - wtm[b]).max())
        for i in range(qd.shape[0]):
            j = int(ta[b, i])
            assert 0 <= j < Db.shape[0], (what, b, i, j)
            if top2[i, 1] - top2[i, 0] > 2 * mg:
                unique += 1
                assert j == wta[b, i], (what, b, i, j, int(wta[b, i]))
            else:
                forced += 1
                assert S[i, j] >= wtm[b, i] - mg, (what, b, i, j)
    say(f"  {what}: argmax equal on {unique} unique (doc, token) pairs, {forced} near-ties valid")


def test_argmax_many_documents_per_wave():
    """The forward with argmax where every wave scores a contiguous range of at least 4
    fixed-length documents (40000 documents of 11 tokens, d=64): scores bit-identical to the
    plain forward, maxima within the margin, argmax as in check_argmax (vectorised)."""
    say("case: argmax, 40000 docs, Nd=11, d=64 bf16")
    c = gen.fixed_corpus(4200, 40000, 32, 11, 64, "bf16")
    s, tm, ta, plain = gpu_argmax(c)
    assert np.array_equal(s.view(np.uint32), plain.view(np.uint32)), "scores differ"
    ws, wtm, wta = oracle.maxsim_argmax(c.Q, c.D, "bf16")
    qd, Dd = dec(c.Q, "bf16"), dec(c.D, "bf16")
    S = (Dd.reshape(-1, Dd.shape[-1]) @ qd.T).reshape(Dd.shape[0], Dd.shape[1], -1)
    S = S.transpose(0, 2, 1)  # [doc, query token, doc token]
    mg = margin_for(64)
    assert np.all(np.abs(tm - wtm) <= mg), np.abs(tm - wtm).max()
    srt = np.sort(S, axis=2)
    unique = srt[:, :, -1] - srt[:, :, -2] > 2 * mg
    assert np.array_equal(ta[unique], wta[unique])
    assert np.all((ta >= 0) & (ta < 11))
    chosen = np.take_along_axis(S, ta[:, :, None].astype(np.int64), axis=2)[:, :, 0]
    assert np.all(chosen[~unique] >= wtm[~unique] - mg)
    say(f"  argmax equal on {int(unique.sum())} unique pairs, {int((~unique).sum())} near-ties valid")


DENSE_Q = [1, 16, 32, 33, 64]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("q_len", DENSE_Q)
def test_argmax_fixed(q_len, dtype):
    say(f"case: argmax fixed q_len={q_len} {dtype} d=128 B=40 Nd=100")
    check_argmax(gen.fixed_corpus(500 + q_len, 40, q_len, 100, 128, dtype), "fixed")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("q_len", [32, 64])
def test_argmax_csr_ragged_and_empty(q_len, dtype):
    lens = np.concatenate([[0, 1, 17, 0, 300, 16, 15], gen.lengths(520 + q_len, 50)])
    say(f"case: argmax CSR q_len={q_len} {dtype} {len(lens)} docs incl. empty")
    check_argmax(gen.csr_corpus(520 + q_len, len(lens), q_len, 128, dtype, lens=lens), "csr")


@pytest.mark.parametrize("d", [64, 256, 768])
def test_argmax_other_d(d):
    say(f"case: argmax d={d} bf16 q_len=32")
    check_argmax(gen.fixed_corpus(540 + d, 30, 32, 70, d, "bf16"), f"d={d}")


@pytest.mark.parametrize("q_len,d,dtype", [(65, 128, "bf16"), (200, 128, "fp16"),
                                           (1024, 128, "bf16"), (100, 128, "fp32"),
                                           (300, 64, "bf16"), (512, 256, "bf16")])
def test_argmax_long_query(q_len, d, dtype):
    say(f"case: argmax long query q_len={q_len} d={d} {dtype}")
    check_argmax(gen.fixed_corpus(560 + q_len, 6, q_len, 260, d, dtype), "long")


def test_argmax_long_query_csr():
    lens = np.array([0, 1, 31, 32, 33, 700, 0, 129])
    say("case: argmax long query CSR q_len=300 bf16")
    check_argmax(gen.csr_corpus(580, len(lens), 300, 128, "bf16", lens=lens), "long csr")


@pytest.mark.parametrize("q_len", [32, 300])
def test_argmax_exact_duplicates_take_lowest_index(q_len):
    """A copy of the argmax token placed later in the document has bit-identical fp32
    similarities: the earlier index must be reported; a document of identical tokens
    reports 0 everywhere."""
    say(f"case: argmax duplicates q_len={q_len}")
    c = gen.fixed_corpus(590 + q_len, 12, q_len, 80, 128, "bf16")
    _, _, wta = oracle.maxsim_argmax(c.Q, c.D, "bf16")
    for b in range(12):
        j0 = int(wta[b, 0])
        if j0 < 79:
            c.D[b, 79] = c.D[b, j0]
    c.D[5] = c.D[5, 3]
    _, _, ta, _ = gpu_argmax(c)
    _, _, wta = oracle.maxsim_argmax(c.Q, c.D, "bf16")
    assert np.all(ta[5] == 0)
    assert np.array_equal(ta[:, 0], wta[:, 0])
    check_argmax(c, "duplicates")


# ---------------------------------------------------------------- backward

def gpu_backward(c, ta, g, grad_dtype="fp32", want_dQ=True, want_dD=True):
    import torch
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[grad_dtype]
    Q, D = dev(c.Q, c.dtype), dev(c.D, c.dtype)
    off = None if c.offsets is None else torch.from_numpy(c.offsets).cuda()
    dQ, dD = ms().maxsim_backward(Q, D, torch.from_numpy(np.ascontiguousarray(ta, np.int32)).cuda(),
                                  torch.from_numpy(np.ascontiguousarray(g, np.float32)).cuda(), off,
                                  want_dQ=want_dQ, want_dD=want_dD, grad_dtype=tdt)
    torch.cuda.synchronize()
    f = lambda t: None if t is None else t.float().cpu().numpy().astype(np.float64)
    return f(dQ), f(dD)


def oracle_grads(c, ta, g):
    """(dQ, dD, M_dQ, M_dD): oracle gradients and the sums of |terms| behind each element."""
    dQ, dD = oracle.maxsim_backward(c.Q, c.D, c.dtype, ta, g, offsets=c.offsets)
    # |x| of a stored value is exact: clear the sign bit of bf16, abs of fp16 / fp32
    absQ = (c.Q & 0x7fff) if c.dtype == "bf16" else np.abs(c.Q)
    absD = (c.D & 0x7fff) if c.dtype == "bf16" else np.abs(c.D)
    mQ, mD = oracle.maxsim_backward(absQ, absD, c.dtype, ta, np.abs(g), offsets=c.offsets)
    return dQ, dD, mQ, mD


def check_bound(got, want, mag, n_terms, grad_dtype, what):
    gam = (n_terms + 1) * U32 / (1 - (n_terms + 1) * U32)
    u = U_GRAD[grad_dtype]
    bound = gam * mag + u * (np.abs(want) + gam * mag) + ETA_GRAD[grad_dtype] + 1e-30
    err = np.abs(got - want)
    assert got.shape == want.shape
    ratio = float((err / bound).max()) if err.size else 0.0
    say(f"  {what}: {err.size} values, max |gpu - oracle| = {err.max():.3e}, "
        f"max error / bound = {ratio:.3f}")
    assert np.all(err <= bound), f"{what}: error above the fp32 summation bound"


def check_backward(c, g, grad_dtype="fp32", what=""):
    _, _, ta = oracle.maxsim_argmax(c.Q, c.D, c.dtype, offsets=c.offsets)
    dQ, dD, mQ, mD = oracle_grads(c, ta, g)
    gQ, gD = gpu_backward(c, ta, g, grad_dtype)
    n_docs = len(g)
    check_bound(gQ, dQ, mQ, n_docs, grad_dtype, f"{what} dQ")
    check_bound(gD, dD, mD, c.Q.shape[0], grad_dtype, f"{what} dD")
    return ta, gQ, gD


@pytest.mark.parametrize("grad_dtype", ["fp32", "same"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_backward_fixed(dtype, grad_dtype):
    gd = dtype if grad_dtype == "same" else "fp32"
    say(f"case: backward fixed {dtype} grads {gd} q_len=32 d=128 B=50 Nd=100")
    c = gen.fixed_corpus(600, 50, 32, 100, 128, dtype)
    g = np.random.default_rng(600).standard_normal(50).astype(np.float32)
    check_backward(c, g, gd, "fixed")


@pytest.mark.parametrize("q_len", [32, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_csr_long_and_empty_documents(dtype, q_len):
    """Documents longer than one inverse-grid segment (256 tokens), empty documents and
    a ragged tail; with 64 query tokens every lane of the chosen-token sets is used."""
    lens = np.concatenate([[0, 2500, 1, 0, 1024, 1025], gen.lengths(610, 40)])
    say(f"case: backward CSR {dtype} q_len={q_len} {len(lens)} docs incl. 2500 tokens and empty")
    c = gen.csr_corpus(610, len(lens), q_len, 128, dtype, lens=lens)
    g = np.random.default_rng(610).standard_normal(len(lens)).astype(np.float32)
    check_backward(c, g, "fp32", "csr")


@pytest.mark.parametrize("q_len,d", [(1024, 128), (1000, 64), (100, 768), (64, 256), (1, 128),
                                       (24, 768), (48, 384)])
def test_backward_query_shapes(q_len, d):
    say(f"case: backward q_len={q_len} d={d} bf16")
    c = gen.fixed_corpus(620 + q_len + d, 5, q_len, 150, d, "bf16")
    g = np.random.default_rng(620).standard_normal(5).astype(np.float32)
    check_backward(c, g, "bf16", f"q={q_len} d={d}")


def test_backward_many_documents_dq_ranges():
    """More documents than dQ ranges (2048): every range sums several documents."""
    say("case: backward 5000 docs q_len=32 Nd=20")
    c = gen.fixed_corpus(630, 5000, 32, 20, 128, "bf16")
    g = np.random.default_rng(630).standard_normal(5000).astype(np.float32)
    check_backward(c, g, "fp32", "5000 docs")


def test_backward_out_of_range_argmax_entries_contribute_nothing():
    say("case: backward with -1 and out-of-range argmax entries")
    c = gen.fixed_corpus(640, 20, 32, 50, 128, "bf16")
    _, _, ta = oracle.maxsim_argmax(c.Q, c.D, "bf16")
    rng = np.random.default_rng(640)
    bad = rng.random(ta.shape) < 0.2
    ta = ta.copy()
    ta[bad] = rng.choice(np.array([-1, -7, 50, 51, 1 << 30], np.int32), size=int(bad.sum()))
    g = rng.standard_normal(20).astype(np.float32)
    dQ, dD, mQ, mD = oracle_grads(c, ta, g)
    gQ, gD = gpu_backward(c, ta, g)
    check_bound(gQ, dQ, mQ, 20, "fp32", "dQ")
    check_bound(gD, dD, mD, 32, "fp32", "dD")


def test_backward_is_deterministic_and_outputs_are_independent():
    say("case: backward run twice; dQ only; dD only")
    lens = gen.lengths(650, 300)
    c = gen.csr_corpus(650, 300, 32, 128, "bf16", lens=lens)
    _, _, ta = oracle.maxsim_argmax(c.Q, c.D, "bf16", offsets=c.offsets)
    g = np.random.default_rng(650).standard_normal(300).astype(np.float32)
    q1, d1 = gpu_backward(c, ta, g)
    q2, d2 = gpu_backward(c, ta, g)
    assert np.array_equal(q1, q2) and np.array_equal(d1, d2)
    q3, none = gpu_backward(c, ta, g, want_dD=False)
    none2, d3 = gpu_backward(c, ta, g, want_dQ=False)
    assert none is None and none2 is None
    assert np.array_equal(q1, q3) and np.array_equal(d1, d3)


def test_backward_zero_rows_are_written():
    """Every row of every document is written: a dD buffer filled with garbage beforehand
    holds exact zeros in the rows no query token chose."""
    import torch
    say("case: backward overwrites unchosen rows")
    c = gen.fixed_corpus(660, 10, 8, 64, 128, "bf16")
    _, _, ta = oracle.maxsim_argmax(c.Q, c.D, "bf16")
    Q, D = dev(c.Q, "bf16"), dev(c.D, "bf16")
    dD = torch.full(D.shape, 7.0, dtype=torch.float32, device="cuda")
    g = torch.ones(10, dtype=torch.float32, device="cuda")
    ms().maxsim_backward(Q, D, torch.from_numpy(ta).cuda(), g, want_dQ=False, dD=dD)
    torch.cuda.synchronize()
    got = dD.cpu().numpy()
    chosen = np.zeros((10, 64), bool)
    for b in range(10):
        chosen[b, ta[b]] = True
    assert np.all(got[~chosen] == 0.0)
    assert np.all(np.abs(got[chosen]).sum(axis=-1) > 0)


def test_autograd_function_matches_oracle():
    """torch.autograd through maxsim(): gradients in the input dtype, from the kernels."""
    import torch
    say("case: autograd MaxSimFunction bf16 q_len=32 B=30")
    c = gen.fixed_corpus(670, 30, 32, 60, 128, "bf16")
    w = np.random.default_rng(670).standard_normal(30).astype(np.float32)
    Q = dev(c.Q, "bf16").requires_grad_(True)
    D = dev(c.D, "bf16").requires_grad_(True)
    scores = ms().maxsim(Q, D)
    (scores * torch.from_numpy(w).cuda()).sum().backward()
    torch.cuda.synchronize()
    assert Q.grad.dtype == torch.bfloat16 and D.grad.dtype == torch.bfloat16
    # the GPU argmax must agree with the oracle's for this comparison to be meaningful
    _, _, ta_gpu, _ = gpu_argmax(c)
    _, _, ta = oracle.maxsim_argmax(c.Q, c.D, "bf16")
    assert np.array_equal(ta_gpu, ta), "near-tie in this seed: choose another"
    dQ, dD, mQ, mD = oracle_grads(c, ta, w)
    check_bound(Q.grad.float().cpu().numpy().astype(np.float64), dQ, mQ, 30, "bf16", "autograd dQ")
    check_bound(D.grad.float().cpu().numpy().astype(np.float64), dD, mD, 32, "bf16", "autograd dD")


@pytest.mark.parametrize("grad_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("layout", ["fixed", "csr"])
def test_backward_no_documents_gives_zero_dQ(layout, grad_dtype):
    """No documents: the loss is an empty sum, so dQ is exactly zero, even where its buffer
    held garbage before the call (dD has no rows)."""
    import torch
    say(f"case: backward with no documents, {layout}, dQ in {grad_dtype}")
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[grad_dtype]
    q_len, d = 32, 128
    Q = torch.ones(q_len, d, dtype=torch.bfloat16, device="cuda")
    if layout == "fixed":
        D, off = torch.empty(0, 16, d, dtype=torch.bfloat16, device="cuda"), None
    else:
        D = torch.empty(0, d, dtype=torch.bfloat16, device="cuda")
        off = torch.zeros(1, dtype=torch.int64, device="cuda")
    ta = torch.empty(0, q_len, dtype=torch.int32, device="cuda")
    g = torch.empty(0, dtype=torch.float32, device="cuda")
    dQ = torch.full((q_len, d), 7.0, dtype=tdt, device="cuda")
    dD = torch.empty(D.shape, dtype=tdt, device="cuda")
    ms().maxsim_backward(Q, D, ta, g, off, grad_dtype=tdt, dQ=dQ, dD=dD)
    torch.cuda.synchronize()
    got = dQ.float().cpu().numpy()
    assert np.all(got == 0.0) and not np.any(np.signbit(got))
