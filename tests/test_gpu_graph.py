"""The scoring path captured in a HIP graph replays to the eager results.

No entry point allocates, clears or copies device memory, or synchronises, on its own:
every buffer (outputs, workspaces) is the caller's, and the allocation-free top-k takes its
scratch from the library's static array. A step of launches can therefore be captured once
and replayed. Each case runs its step eagerly, captures it, and replays the graph three
times, with the outputs refilled with a sentinel by eager work and a synchronisation
between replays; every replay must reproduce the eager outputs bit for bit.
"""
import numpy as np
import pytest

import gen
from gpu_util import ms, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ms()
    yield
    torch.cuda.empty_cache()


def _bits(t):
    a = t.detach().cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.float32 else a.copy()


def _fill(outs):
    import torch
    for t in outs:
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)
    torch.cuda.synchronize()


def step_score_topk():
    """Headline shape in miniature: one query, fixed documents, top-100 with a workspace."""
    import torch
    c = gen.fixed_corpus(21, 3000, 32, 77, 128, "bf16")
    Q, D = gen.to_device(c.Q, "bf16"), gen.to_device(c.D, "bf16")
    scores = torch.empty(c.n_docs, dtype=torch.float32, device="cuda")
    k = 100
    vals = torch.empty(k, dtype=torch.float32, device="cuda")
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(16, ms().topk_workspace_size(c.n_docs, 1, k)), dtype=torch.uint8,
                     device="cuda")

    def step():
        ms().maxsim_score_fixed(Q, D, out=scores)
        ms().maxsim_topk(scores, k, out_scores=vals, out_index=idx, workspace=ws)
    return step, [scores, vals, idx]


def step_score_topk_no_alloc():
    """CSR documents, then the top-k entry point that allocates nothing."""
    import torch
    c = gen.csr_corpus(22, 3000, 32, 128, "bf16")
    Q, D = gen.to_device(c.Q, "bf16"), gen.to_device(c.D, "bf16")
    off = torch.from_numpy(c.offsets).cuda()
    scores = torch.empty(c.n_docs, dtype=torch.float32, device="cuda")
    k = 64
    vals = torch.empty(k, dtype=torch.float32, device="cuda")
    idx = torch.empty(k, dtype=torch.int32, device="cuda")

    def step():
        ms().maxsim_score(Q, D, off, out=scores)
        ms().maxsim_topk_no_alloc(scores, k, vals, idx)
    return step, [scores, vals, idx]


def step_long_query_and_batch():
    """The query-tiled kernel (300 tokens) and both several-query kernels."""
    import torch
    c = gen.fixed_corpus(23, 1500, 300 + 256 + 1024, 77, 128, "bf16")
    Qall = gen.to_device(c.Q, "bf16")
    D = gen.to_device(c.D, "bf16")
    Ql, Q8, Q32 = Qall[:300], Qall[300:556].view(8, 32, 128), Qall[556:].view(32, 32, 128)
    s1 = torch.empty(c.n_docs, dtype=torch.float32, device="cuda")
    s8 = torch.empty(8, c.n_docs, dtype=torch.float32, device="cuda")
    s32 = torch.empty(32, c.n_docs, dtype=torch.float32, device="cuda")

    def step():
        ms().maxsim_score_fixed(Ql, D, out=s1)
        ms().maxsim_score_batch(Q8, D, out=s8)
        ms().maxsim_score_batch(Q32, D, out=s32)
    return step, [s1, s8, s32]


def step_training():
    """Forward with per-token argmax, then dQ and dD in bf16 with a caller workspace."""
    import torch
    B, nd, q, d = 1200, 77, 32, 128
    c = gen.fixed_corpus(24, B, q, nd, d, "bf16")
    Q, D = gen.to_device(c.Q, "bf16"), gen.to_device(c.D, "bf16")
    g = torch.from_numpy(np.random.default_rng(24).standard_normal(B).astype(np.float32)).cuda()
    out = torch.empty(B, dtype=torch.float32, device="cuda")
    tmax = torch.empty(B, q, dtype=torch.float32, device="cuda")
    targ = torch.empty(B, q, dtype=torch.int32, device="cuda")
    dQ = torch.empty(q, d, dtype=torch.bfloat16, device="cuda")
    dD = torch.empty(D.shape, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(16, ms().backward_workspace_size(q, d, B)), dtype=torch.uint8,
                     device="cuda")

    def step():
        ms().maxsim_score_argmax(Q, D, out=out, tok_max=tmax, tok_arg=targ)
        ms().maxsim_backward(Q, D, targ, g, None, want_dQ=True, want_dD=True,
                             grad_dtype=torch.bfloat16, dQ=dQ, dD=dD, workspace=ws)
    return step, [out, tmax, targ, dQ.view(torch.int16), dD.view(torch.int16)]


def step_pq():
    """PQ tables built on the device, then fused lookup scoring over CSR codes."""
    import torch
    C = torch.from_numpy(gen.codebook(25)).cuda()
    Q = gen.to_device(gen.tokens(25, gen.S_QUERY, 0, 32, 128, "bf16"), "bf16")
    off_h = gen.csr_offsets(gen.lengths(25, 2000, 70.0, 0.5, 8, 512))
    codes = torch.from_numpy(gen.codes(25, int(off_h[-1]))).cuda()
    off = torch.from_numpy(off_h).cuda()
    T = torch.empty(32, 16, 256, dtype=torch.float32, device="cuda")
    out = torch.empty(2000, dtype=torch.float32, device="cuda")

    def step():
        ms().maxsim_pq_tables(Q, C, T=T)
        ms().maxsim_score_pq(T, codes, off, out=out)
    return step, [T, out]


STEPS = {"score+topk": step_score_topk, "csr+topk-no-alloc": step_score_topk_no_alloc,
         "long-query+batch": step_long_query_and_batch, "training": step_training,
         "pq": step_pq}


@pytest.mark.parametrize("name", list(STEPS))
def test_graph_replays_match_eager(name):
    import torch
    say(f"case: graph capture {name}")
    step, outs = STEPS[name]()
    _fill(outs)
    step()
    torch.cuda.synchronize()
    eager = [_bits(t) for t in outs]
    # warm up on a side stream (default priority), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        _fill(outs)
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, t) in enumerate(zip(eager, outs)):
            assert np.array_equal(a, _bits(t)), f"{name}: replay {r}, output {k} differs"
