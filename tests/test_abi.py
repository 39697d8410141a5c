"""The C-ABI library: it loads, exports every declared entry point, and rejects bad
arguments with the documented status codes before touching the GPU (CPU-only)."""
import ctypes
import os
import re

import pytest
import torch

import maxsim_scoring_fwd_amd as ms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "maxsim.h")
CALIB_HEADER = os.path.join(ROOT, "include", "maxsim_calib.h")

OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, LAUNCH, DEVICE = 0, -1, -2, -3, -4, -5, -6, -7
P = 0x10000  # a 16-byte aligned stand-in address; never dereferenced by these calls


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ms.LIB_PATH):
        from maxsim_scoring_fwd_amd import build
        build.build()
    return ms.lib()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(maxsim_\w+)\s*\(", text, re.M)))


def test_header_declares_entry_points():
    names = declared_functions()
    for f in ("maxsim_score", "maxsim_score_fixed", "maxsim_score_i8", "maxsim_pq_tables",
              "maxsim_score_pq", "maxsim_status_string", "maxsim_version", "maxsim_score_argmax",
              "maxsim_backward", "maxsim_backward_workspace_size", "maxsim_score_batch",
              "maxsim_topk", "maxsim_topk_workspace_size"):
        assert f in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {ms.LIB_PATH}").read()
    exported = set(re.findall(r" T (maxsim_\w+)", out))
    assert set(declared_functions()) <= exported


def test_calibration_symbols_are_exported(L):
    names = declared_functions(CALIB_HEADER)
    assert {"maxsim_calib_read", "maxsim_calib_copy", "maxsim_calib_mfma",
            "maxsim_calib_write", "maxsim_calib_valu", "maxsim_calib_mix",
            "maxsim_calib_lds"} <= set(names)
    out = os.popen(f"nm -D --defined-only {ms.LIB_PATH}").read()
    assert set(names) <= set(re.findall(r" T (maxsim_\w+)", out))


def test_calibration_argument_checks(L):
    ops = ctypes.c_double(0.0)
    f = L.maxsim_calib_mfma
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    assert f(0, 10, 1, None, ctypes.addressof(ops), None) == NULL
    assert f(4, 10, 1, P, ctypes.addressof(ops), None) == SHAPE
    assert f(0, 0, 1, P, ctypes.addressof(ops), None) == SHAPE
    assert f(0, 10, 9, P, ctypes.addressof(ops), None) == SHAPE
    v, mx, lds = L.maxsim_calib_valu, L.maxsim_calib_mix, L.maxsim_calib_lds
    v.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    mx.argtypes = [ctypes.c_int] + v.argtypes
    lds.argtypes = v.argtypes
    assert v(10, 1, None, ctypes.addressof(ops), None) == NULL
    assert v(0, 1, P, ctypes.addressof(ops), None) == SHAPE
    assert mx(3, 10, 2, P, ctypes.addressof(ops), None) == SHAPE  # 0, 1, 2, 4 or 8 per MFMA
    assert mx(4, 10, 9, P, ctypes.addressof(ops), None) == SHAPE
    assert lds(2, 10, P, ctypes.addressof(ops), None) == SHAPE    # pattern 0 or 1
    assert lds(0, 10, P, None, None) == NULL


def test_no_torch_in_signatures():
    text = open(HEADER).read()
    assert "torch" not in text.lower().replace("caller-allocated", "")
    assert "at::" not in text and "Tensor" not in text


def test_status_strings_and_version(L):
    for s in (OK, NULL, SHAPE, DTYPE, ALIGN, UNSUP, LAUNCH, DEVICE):
        assert len(L.maxsim_status_string(s)) >= 2
    assert L.maxsim_version() >= 100


def score(L, Q=P, q_len=32, D=P, off=P, n=10, d=128, dt=0, out=P):
    return L.maxsim_score(Q, q_len, D, off, n, d, dt, out, None)


def fixed(L, Q=P, q_len=32, D=P, n=10, nd=128, lens=None, d=128, dt=0, out=P):
    return L.maxsim_score_fixed(Q, q_len, D, n, nd, lens, d, dt, out, None)


def test_dense_argument_errors(L):
    assert score(L, Q=None) == NULL
    assert score(L, D=None) == NULL
    assert score(L, out=None) == NULL
    assert score(L, off=None) == NULL
    assert score(L, q_len=0) == SHAPE
    assert score(L, q_len=1025) == SHAPE
    assert score(L, d=48) == SHAPE
    assert score(L, d=16) == SHAPE
    assert score(L, d=1056) == SHAPE
    assert score(L, n=-1) == SHAPE
    assert score(L, dt=3) == DTYPE
    assert score(L, dt=-1) == DTYPE
    assert score(L, Q=P + 2) == ALIGN
    assert score(L, D=P + 8) == ALIGN
    assert score(L, out=P + 2) == ALIGN
    assert score(L, off=P + 4) == ALIGN
    assert fixed(L, nd=0) == SHAPE
    assert fixed(L, lens=P + 2) == ALIGN
    assert fixed(L, Q=None) == NULL


def test_zero_docs_is_a_no_op(L):
    assert score(L, n=0) == OK
    assert fixed(L, n=0) == OK
    assert L.maxsim_score_i8(P, P, 32, P, P, None, 0, 16, 128, P, None, None, None) == OK
    assert L.maxsim_score_pq(P, 32, 16, 256, P, None, 0, 16, P, None) == OK


def test_i8_argument_errors(L):
    f = lambda **k: L.maxsim_score_i8(k.get("Q", P), k.get("qs", P), k.get("q_len", 32),
                                      k.get("D", P), k.get("ds", P), k.get("off", None),
                                      k.get("n", 5), k.get("nd", 16), k.get("d", 128),
                                      k.get("out", P), k.get("tm", None), k.get("ta", None), None)
    assert f(d=96) == SHAPE
    assert f(d=32) == SHAPE
    assert f(nd=0) == SHAPE
    assert f(q_len=0) == SHAPE
    assert f(Q=None) == NULL
    assert f(qs=None) == NULL
    assert f(ds=None) == NULL
    assert f(tm=P) == NULL  # tok_max without tok_arg
    assert f(D=P + 4) == ALIGN
    assert f(qs=P + 1) == ALIGN
    assert f(off=P + 4) == ALIGN


def test_pq_argument_errors(L):
    t = lambda **k: L.maxsim_pq_tables(k.get("Q", P), k.get("q_len", 32), k.get("dt", 0),
                                       k.get("C", P), k.get("M", 16), k.get("K", 256),
                                       k.get("dsub", 8), k.get("T", P), None)
    assert t(K=128) == UNSUP
    assert t(dt=7) == DTYPE
    assert t(M=3, dsub=8) == SHAPE  # d = 24
    assert t(dsub=33) == SHAPE
    assert t(C=None) == NULL
    assert t(T=P + 4) == ALIGN
    s = lambda **k: L.maxsim_score_pq(k.get("T", P), k.get("q_len", 32), k.get("M", 16),
                                      k.get("K", 256), k.get("codes", P), k.get("off", None),
                                      k.get("n", 5), k.get("nd", 16), k.get("out", P), None)
    assert s(K=16) == UNSUP
    assert s(M=8) == UNSUP
    assert s(q_len=65) == UNSUP
    assert s(nd=0) == SHAPE
    assert s(codes=None) == NULL
    assert s(codes=P + 8) == ALIGN


def test_argmax_argument_errors(L):
    f = lambda **k: L.maxsim_score_argmax(k.get("Q", P), k.get("q_len", 32), k.get("D", P),
                                          k.get("off", None), k.get("n", 5), k.get("nd", 16),
                                          k.get("d", 128), k.get("dt", 0), k.get("out", P),
                                          k.get("tm", P), k.get("ta", P), None)
    assert f(tm=None) == NULL
    assert f(ta=None) == NULL
    assert f(out=None) == NULL
    assert f(nd=0) == SHAPE
    assert f(d=48) == SHAPE
    assert f(dt=5) == DTYPE
    assert f(tm=P + 2) == ALIGN
    assert f(off=P + 4) == ALIGN
    assert f(n=0) == OK


def test_batch_argument_errors(L):
    f = lambda **k: L.maxsim_score_batch(k.get("Q", P), k.get("n_q", 4), k.get("q_len", 32),
                                         k.get("D", P), k.get("off", None), k.get("n", 5),
                                         k.get("nd", 16), k.get("d", 128), k.get("dt", 0),
                                         k.get("out", P), None)
    assert f(n_q=0) == SHAPE
    assert f(nd=0) == SHAPE
    assert f(q_len=0) == SHAPE
    assert f(Q=None) == NULL
    assert f(out=P + 2) == ALIGN
    assert f(off=P + 4) == ALIGN
    assert f(d=768) == UNSUP          # 1536-byte rows: no query-tiled kernel
    assert f(dt=2, d=256) == UNSUP    # fp32 rows of 1 KiB
    assert f(n=0) == OK


def test_topk_argument_errors_and_workspace(L):
    f = lambda **k: L.maxsim_topk(k.get("S", P), k.get("n", 100000), k.get("rows", 1),
                                  k.get("k", 100), k.get("vo", P), k.get("io", P),
                                  k.get("ws", P), k.get("wsb", 1 << 30), None)
    assert f(k=0) == SHAPE and f(k=1025) == SHAPE and f(n=0) == SHAPE and f(rows=0) == SHAPE
    assert f(S=None) == NULL and f(io=None) == NULL
    assert f(ws=None) == NULL              # 100000 scores need the workspace
    assert f(wsb=8) == SHAPE               # too small
    assert f(S=P + 2) == ALIGN and f(ws=P + 4) == ALIGN
    w = L.maxsim_topk_workspace_size
    assert w(2048, 1, 100) == 0            # one chunk: no workspace
    # k <= 128: one sorted run of 128 keys per 2048 scores; a second region when the runs
    # need two or more merge passes (more than 64 runs)
    assert w(100000, 1, 100) == 49 * 128 * 8
    assert w(100000, 32, 10) == 49 * 128 * 8 * 32
    assert w(5000000, 1, 128) == (2442 + 39) * 128 * 8
    # k > 128: chunks of 2048 sorted in LDS, k kept per chunk, level by level
    assert w(100000, 1, 129) == (49 + 4) * 129 * 8
    assert w(100000, 1, 1024) == (49 + 25) * 1024 * 8
    assert w(0, 1, 10) == 0 and w(10, 1, 0) == 0


def bwd(L, **k):
    return L.maxsim_backward(k.get("Q", P), k.get("q_len", 32), k.get("D", P), k.get("off", None),
                             k.get("n", 5), k.get("nd", 16), k.get("d", 128), k.get("dt", 0),
                             k.get("ta", P), k.get("g", P), k.get("dQ", P), k.get("dD", P),
                             k.get("gdt", 2), k.get("ws", P), k.get("wsb", 1 << 30), None)


def test_backward_argument_errors(L):
    assert bwd(L, ta=None) == NULL
    assert bwd(L, g=None) == NULL
    assert bwd(L, ws=None) == NULL          # dQ needs the workspace
    assert bwd(L, gdt=1) == DTYPE           # bf16 data, fp16 gradients
    assert bwd(L, dt=9) == DTYPE
    assert bwd(L, q_len=1025) == SHAPE
    assert bwd(L, nd=0) == SHAPE
    assert bwd(L, wsb=1024) == SHAPE        # workspace too small
    assert bwd(L, dD=P + 8) == ALIGN
    assert bwd(L, ws=P + 4) == ALIGN
    assert bwd(L, n=0, dQ=None) == OK       # no documents: no dD rows to write
    assert bwd(L, n=0, dQ=None, D=None, ta=None, g=None) == OK  # empty arrays may be NULL
    assert bwd(L, n=1, dQ=None, D=None) == NULL
    assert bwd(L, dQ=None, dD=None) == OK   # nothing asked for


def test_backward_workspace_size(L):
    f = L.maxsim_backward_workspace_size
    # 32 x 128 dQ: one block of 4096 elements, 2048 document ranges of fp32 partial sums
    assert f(32, 128, 100000) == 2048 * 32 * 128 * 4
    assert f(32, 128, 10) == 10 * 32 * 128 * 4      # never more ranges than documents
    assert f(1024, 128, 175000) == 64 * 1024 * 128 * 4
    assert f(0, 128, 10) == 0 and f(32, 48, 10) == 0 and f(32, 128, 0) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
def test_valid_call_without_gpu_reports_device_error(L):
    assert score(L) == DEVICE
    assert fixed(L) == DEVICE
    # no documents but dQ set: dQ is zeroed on the device, so the device is needed
    assert bwd(L, n=0) == DEVICE


def test_python_binding_refuses_host_tensors(L):
    Q = torch.zeros(32, 128, dtype=torch.bfloat16)
    D = torch.zeros(4, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ms.maxsim_score_fixed(Q, D, out=torch.zeros(4))
