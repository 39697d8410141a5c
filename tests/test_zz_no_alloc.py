"""The allocation-free top-k entry point (maxsim_topk_no_alloc) against maxsim_topk: the
same selection on the same scores, bit for bit, on consecutive calls that share the static
scratch array (the second with a smaller input, so stale runs of the first stay in it), and
a clear error where the call needs more than the array holds."""
import ctypes

import numpy as np
import pytest

from gpu_util import ms, say

pytestmark = pytest.mark.gpu


def scores(seed, rows, n):
    rng = np.random.default_rng(seed)
    S = (rng.integers(-3000, 3000, size=(rows, n)) / 64.0).astype(np.float32)  # many ties
    S[rng.random((rows, n)) < 0.01] = -np.inf
    return S


def call_both(S, k):
    import torch
    m = ms()
    St = torch.from_numpy(np.ascontiguousarray(S)).cuda()
    rows, n = S.shape
    ws = torch.empty(max(16, m.topk_workspace_size(n, rows, k)), dtype=torch.uint8, device="cuda")
    v0, i0 = m.maxsim_topk(St, k, workspace=ws)
    v1 = torch.full((rows, k), 7.0, dtype=torch.float32, device="cuda")
    i1 = torch.full((rows, k), 7, dtype=torch.int32, device="cuda")
    # through the C-ABI directly, on the current stream
    rc = m.lib().maxsim_topk_no_alloc(St.data_ptr(), n, rows, k, v1.data_ptr(), i1.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert rc == 0, m.lib().maxsim_status_string(rc)
    torch.cuda.synchronize()
    return (v0.cpu().numpy(), i0.cpu().numpy()), (v1.cpu().numpy(), i1.cpu().numpy())


@pytest.mark.parametrize("cases", [
    [(4, 1_000_000, 100), (1, 5000, 10)],       # run path: many runs, then few
    [(2, 300_000, 1000), (3, 2100, 200)],       # LDS levels
    [(32, 100_000, 128), (1, 100_000, 100)],    # a batch, then the single-query shape
])
def test_no_alloc_matches_topk_twice(cases):
    for j, (rows, n, k) in enumerate(cases):
        say(f"case: no-alloc top-{k} of {rows} x {n} (call {j + 1} of {len(cases)})")
        S = scores(900 + 7 * j + rows + k, rows, n)
        (v0, i0), (v1, i1) = call_both(S, k)
        assert np.array_equal(i1, i0) and np.array_equal(v1.view(np.uint32), v0.view(np.uint32))


def test_no_alloc_rejects_what_the_scratch_cannot_hold():
    import torch
    m = ms()
    cap = m.topk_scratch_bytes()
    assert cap == 8 << 20
    rows, n, k = 65_535, 4096, 128  # 2 runs of 1 KiB per row: 128 MiB of runs
    assert m.topk_workspace_size(n, rows, k) > cap
    say("case: no-alloc top-k beyond the scratch size")
    rc = m.lib().maxsim_topk_no_alloc(ctypes.c_void_p(16), n, rows, k, ctypes.c_void_p(16),
                                      ctypes.c_void_p(16), None)
    assert rc == -8  # MAXSIM_ERR_SCRATCH, before anything is enqueued
