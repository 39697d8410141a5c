"""Host-side argument checks of the Python binding (CPU only). The library takes every type
from its arguments (the storage type from Q, offsets as int64, argmax as int32 ...) and
cannot see a tensor's dtype, so a wrong dtype or shape must be refused before any pointer
reaches it. These calls use host tensors: the checks fire before the device is touched."""
import pytest
import torch

import maxsim_scoring_fwd_amd as ms

bf, f32, i32, i64 = torch.bfloat16, torch.float32, torch.int32, torch.int64


def Z(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def refuses(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_csr_score_checks():
    Q, D, off = Z(32, 128), Z(100, 128), torch.tensor([0, 50, 100], dtype=i64)
    refuses(lambda: ms.maxsim_score(Z(32, 128, dtype=f32), D, off), "D must have dtype")
    refuses(lambda: ms.maxsim_score(Q, D, off.to(i32)), "doc_offsets must have dtype")
    refuses(lambda: ms.maxsim_score(Q, Z(100, 64), off), "d = 64")
    refuses(lambda: ms.maxsim_score(Q, D, None), "needs doc_offsets")
    refuses(lambda: ms.maxsim_score(Q.to(torch.int8), D, off), "Q must have dtype")
    refuses(lambda: ms.maxsim_score(Q, D, off, out=Z(2, dtype=torch.float64)), "out must have dtype")
    refuses(lambda: ms.maxsim_score(Q, D, off, out=Z(3, dtype=f32)), "2 elements")


def test_fixed_score_checks():
    Q, D = Z(32, 128), Z(4, 16, 128)
    refuses(lambda: ms.maxsim_score_fixed(Q, Z(4, 16, 128, dtype=torch.float16)), "D must have dtype")
    refuses(lambda: ms.maxsim_score_fixed(Q, Z(64, 128)), "3 dimensions")
    refuses(lambda: ms.maxsim_score_fixed(Q, D, Z(4, dtype=i64)), "doc_lens must have dtype")
    refuses(lambda: ms.maxsim_score_fixed(Q, D, Z(5, dtype=i32)), "4 elements")


def test_i8_checks():
    Q, qs = Z(32, 128, dtype=torch.int8), Z(32, dtype=f32)
    D, ds = Z(4, 16, 128, dtype=torch.int8), Z(64, dtype=f32)
    refuses(lambda: ms.maxsim_score_i8(Q.to(bf), qs, D, ds), "Q must have dtype")
    refuses(lambda: ms.maxsim_score_i8(Q, qs, D.to(torch.uint8), ds), "D must have dtype")
    refuses(lambda: ms.maxsim_score_i8(Q, qs.to(torch.float64), D, ds), "q_scale must have dtype")
    refuses(lambda: ms.maxsim_score_i8(Q, qs, D, Z(63, dtype=f32)), "64 elements")
    refuses(lambda: ms.maxsim_score_i8(Q, qs, Z(64, 128, dtype=torch.int8), ds,
                                       torch.tensor([0, 64], dtype=i32)), "doc_offsets must have")


def test_argmax_batch_backward_checks():
    Q, D = Z(32, 128), Z(4, 16, 128)
    refuses(lambda: ms.maxsim_score_argmax(Q, D, tok_arg=Z(4, 32, dtype=i64)), "tok_arg must have")
    refuses(lambda: ms.maxsim_score_argmax(Q, D, tok_max=Z(4, 31, dtype=f32)), "shape")
    refuses(lambda: ms.maxsim_score_batch(Z(2, 32, 128), Z(4, 16, 64)), "d = 64")
    refuses(lambda: ms.maxsim_score_batch(Q, D), "3 dimensions")
    ta, g = Z(4, 32, dtype=i32), Z(4, dtype=f32)
    refuses(lambda: ms.maxsim_backward(Q, D, ta.to(i64), g), "tok_arg must have")
    refuses(lambda: ms.maxsim_backward(Q, D, ta, g.to(bf)), "grad_out must have")
    refuses(lambda: ms.maxsim_backward(Q, D, ta, Z(5, dtype=f32)), "4 elements")
    refuses(lambda: ms.maxsim_backward(Q, D, ta, g, dQ=Z(32, 128, dtype=bf)), "dQ must have")
    refuses(lambda: ms.maxsim_backward(Q, D, ta, g, dD=Z(4, 16, 64, dtype=f32)), "dD must have shape")
    refuses(lambda: ms.maxsim_backward(Q, D, ta, g, workspace=Z(16, dtype=f32)), "workspace must")


def test_pq_and_topk_checks():
    Q, C = Z(32, 128), Z(16, 256, 8, dtype=f32)
    refuses(lambda: ms.maxsim_pq_tables(Q, C.to(bf)), "C must have dtype")
    refuses(lambda: ms.maxsim_pq_tables(Z(32, 64), C), "M \\* dsub")
    T, codes = Z(32, 16, 256, dtype=f32), Z(100, 16, dtype=torch.uint8)
    refuses(lambda: ms.maxsim_score_pq(T, codes.to(torch.int8), nd=10), "codes must have dtype")
    refuses(lambda: ms.maxsim_score_pq(T, Z(100, 8, dtype=torch.uint8), nd=10), "subspaces")
    refuses(lambda: ms.maxsim_score_pq(T, codes), "nd >= 1")
    refuses(lambda: ms.maxsim_score_pq(T.to(bf), codes, nd=10), "T must have dtype")
    S = Z(1000, dtype=f32)
    refuses(lambda: ms.maxsim_topk(S.to(bf), 10), "scores must have dtype")
    refuses(lambda: ms.maxsim_topk(S, 10, out_index=Z(10, dtype=i64)), "out_index must have")
    refuses(lambda: ms.maxsim_topk(S, 10, out_scores=Z(11, dtype=f32)), "10 elements")
