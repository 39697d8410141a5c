"""Helpers for the GPU parity tests: move generated inputs to the device, call the
library through its C-ABI binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import gen
import oracle

TOL = 1e-4      # |gpu - oracle| for bf16 / fp16 / fp32 storage with fp32 accumulation
PQ_TOL = 1e-3   # PQ path against an oracle using the same codebook and codes


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ms():
    import maxsim_scoring_fwd_amd
    maxsim_scoring_fwd_amd.lib()  # raises if the library is not built
    return maxsim_scoring_fwd_amd


def dev_fixed(c, device="cuda", chunk_docs=None):
    import torch
    Q = gen.to_device(c.Q, c.dtype, device)
    D = gen.to_device(c.D, c.dtype, device)
    return Q, D


def gpu_scores_fixed(c, doc_lens=None):
    import torch
    Q, D = dev_fixed(c)
    lens = None if doc_lens is None else torch.from_numpy(np.asarray(doc_lens, np.int32)).cuda()
    out = ms().maxsim_score_fixed(Q, D, lens)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def gpu_scores_csr(c):
    import torch
    Q = gen.to_device(c.Q, c.dtype)
    D = gen.to_device(c.D, c.dtype)
    off = torch.from_numpy(c.offsets).cuda()
    out = ms().maxsim_score(Q, D, off)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def compare(got: np.ndarray, want: np.ndarray, tol: float = TOL, what: str = ""):
    """Element-wise comparison; -inf must match -inf exactly."""
    assert got.shape == want.shape, (got.shape, want.shape)
    ninf_w = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), ninf_w), f"{what}: -inf pattern differs"
    assert np.all(np.isfinite(got[~ninf_w])), f"{what}: non-finite GPU score"
    err = np.abs(got[~ninf_w] - want[~ninf_w])
    mx = float(err.max()) if err.size else 0.0
    say(f"  {what}: {got.size} scores, max |gpu - oracle| = {mx:.3e}")
    assert mx <= tol, f"{what}: max error {mx} > {tol}"
    return mx


def topk_agree(got: np.ndarray, want: np.ndarray, k: int, tie: float = 2 * TOL):
    """Top-k by score (descending, then index ascending): identical except where oracle
    scores within `tie` of each other make the order ambiguous."""
    og = np.lexsort((np.arange(len(got)), -got))[:k]
    ow = np.lexsort((np.arange(len(want)), -want))[:k]
    if np.array_equal(og, ow):
        return 0
    # allowed only where the oracle scores of differing positions are tied
    kth = want[ow[-1]]
    for a, b in zip(og, ow):
        if a != b:
            assert abs(want[a] - want[b]) <= tie or abs(want[a] - kth) <= tie, (a, b)
    return 1
