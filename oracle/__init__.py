"""MaxSim oracle (float64, CPU) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package. The GPU library never calls it, and it shares no code with the GPU path.

Definition followed (TileMaxSim deep reading, section 1; Flash-MaxSim abstract):
score_b = sum over query tokens i of max over document tokens j of <q_i, d_j>, on
the stored values, accumulated in float64. The backward pass (Flash-MaxSim
abstract: training backward through the forward argmax) is the gradient of
sum_b g_b * score_b: dQ[i] = sum_b g_b d_{b,j*(b,i)}, dD[b,j] = g_b * sum of the q_i
whose argmax is j. The C source states every reading
taken where the pages are silent (padding, empty documents, INT8 scale formula,
PQ table layout).

Pins: tests/test_oracle_pins.py (brute force, closed forms, invariants, golden
hand-worked examples) and tests/test_oracle_mutants.py (planted mistakes must
fail a pin).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "maxsim_oracle.c")
_SO = os.path.join(_HERE, "_maxsim_oracle.so")

DTYPES = {"bf16": 0, "fp16": 1, "fp32": 2}
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def compile_oracle(src: str, so: str) -> str:
    """Compile an oracle source file into a shared library (used by build and by mutant tests)."""
    tmp = so + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, src, "-lm", "-lpthread"])
    os.replace(tmp, so)
    return so


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(SRC):
        compile_oracle(SRC, _SO)
    return _SO


def _bind(lib):
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.oracle_maxsim_csr.argtypes = [vp, i32, vp, vp, i64, i32, i32, vp, i32]
    lib.oracle_maxsim_fixed.argtypes = [vp, i32, vp, i64, i32, vp, i32, i32, vp, i32]
    lib.oracle_maxsim_i8.argtypes = [vp, vp, i32, vp, vp, vp, i64, i32, i32, vp, vp, vp, i32]
    lib.oracle_pq_tables.argtypes = [vp, i32, i32, vp, i32, i32, i32, vp]
    lib.oracle_maxsim_pq.argtypes = [vp, i32, i32, i32, vp, vp, i64, i32, vp, i32]
    lib.oracle_maxsim_argmax.argtypes = [vp, i32, vp, vp, i64, i32, i32, i32, vp, vp, vp, i32]
    lib.oracle_maxsim_backward.argtypes = [vp, i32, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp]
    for f in ("oracle_maxsim_csr", "oracle_maxsim_fixed", "oracle_maxsim_i8", "oracle_pq_tables",
              "oracle_maxsim_pq", "oracle_maxsim_argmax", "oracle_maxsim_backward"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def host_threads() -> int:
    """Host cores this process may run on (its CPU affinity), or OMP_NUM_THREADS where the
    environment sets a smaller share."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def _threads(n):
    return n if n else host_threads()


def _c(a, dt=None):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


class Oracle:
    """ctypes front end of one compiled oracle library (the real one, or a test mutant)."""

    def __init__(self, so_path: str):
        self.lib = _bind(ctypes.CDLL(so_path))

    def _rc(self, rc, what):
        if rc != 0:
            raise ValueError(f"oracle: {what} rejected its arguments")

    def maxsim_fixed(self, Q, D, dtype: str, doc_lens=None, nthreads=None) -> np.ndarray:
        """Q [q_len, d], D [n_docs, nd, d] storage arrays; returns float64 [n_docs]."""
        Q, D = _c(Q), _c(D)
        n_docs, nd, d = D.shape
        out = np.empty(n_docs, dtype=np.float64)
        lens = _c(doc_lens, np.int32)
        self._rc(self.lib.oracle_maxsim_fixed(_ptr(Q), Q.shape[0], _ptr(D), n_docs, nd, _ptr(lens),
                                              d, DTYPES[dtype], _ptr(out), _threads(nthreads)),
                 "maxsim_fixed")
        return out

    def maxsim_csr(self, Q, D, offsets, dtype: str, nthreads=None) -> np.ndarray:
        """Q [q_len, d], D [n_tokens, d], offsets int64 [n_docs+1]; returns float64 [n_docs]."""
        Q, D, off = _c(Q), _c(D), _c(offsets, np.int64)
        n_docs = len(off) - 1
        out = np.empty(n_docs, dtype=np.float64)
        self._rc(self.lib.oracle_maxsim_csr(_ptr(Q), Q.shape[0], _ptr(D), _ptr(off), n_docs,
                                            Q.shape[1], DTYPES[dtype], _ptr(out),
                                            _threads(nthreads)), "maxsim_csr")
        return out

    def maxsim_i8(self, Q, q_scale, D, d_scale, offsets=None, nthreads=None):
        """INT8 scoring. Fixed layout when offsets is None (D [n_docs, nd, d], d_scale
        [n_docs, nd]); CSR otherwise. Returns (scores f64 [n_docs], tok_max f32 [n_docs, q_len],
        tok_arg i32 [n_docs, q_len])."""
        Q, qs, D, ds = _c(Q, np.int8), _c(q_scale, np.float32), _c(D, np.int8), _c(d_scale,
                                                                                  np.float32)
        q_len, d = Q.shape
        if offsets is None:
            n_docs, nd = D.shape[0], D.shape[1]
            off = None
        else:
            off = _c(offsets, np.int64)
            n_docs, nd = len(off) - 1, 0
        out = np.empty(n_docs, dtype=np.float64)
        tm = np.empty((n_docs, q_len), dtype=np.float32)
        ta = np.empty((n_docs, q_len), dtype=np.int32)
        self._rc(self.lib.oracle_maxsim_i8(_ptr(Q), _ptr(qs), q_len, _ptr(D), _ptr(ds), _ptr(off),
                                           n_docs, nd, d, _ptr(out), _ptr(tm), _ptr(ta),
                                           _threads(nthreads)), "maxsim_i8")
        return out, tm, ta

    @staticmethod
    def _layout(D, offsets):
        """(n_docs, nd, offsets) for fixed documents D [n_docs, nd, d] or CSR tokens D [n, d]."""
        if offsets is None:
            return D.shape[0], D.shape[1], None
        off = _c(offsets, np.int64)
        return len(off) - 1, 0, off

    def maxsim_argmax(self, Q, D, dtype: str, offsets=None, nthreads=None):
        """Scores with per-token maxima and argmax (lowest index among equal maxima).
        Fixed layout when offsets is None (D [n_docs, nd, d]), else CSR (D [n_tokens, d]).
        Returns (scores f64 [n_docs], tok_max f64 [n_docs, q_len], tok_arg i32 [n_docs, q_len])."""
        Q, D = _c(Q), _c(D)
        n_docs, nd, off = self._layout(D, offsets)
        q_len, d = Q.shape
        out = np.empty(n_docs, dtype=np.float64)
        tm = np.empty((n_docs, q_len), dtype=np.float64)
        ta = np.empty((n_docs, q_len), dtype=np.int32)
        self._rc(self.lib.oracle_maxsim_argmax(_ptr(Q), q_len, _ptr(D), _ptr(off), n_docs, nd, d,
                                               DTYPES[dtype], _ptr(out), _ptr(tm), _ptr(ta),
                                               _threads(nthreads)), "maxsim_argmax")
        return out, tm, ta

    def maxsim_backward(self, Q, D, dtype: str, tok_arg, grad, offsets=None, want_dQ=True,
                        want_dD=True):
        """Gradients of sum_b grad[b] * score_b for the argmax tok_arg [n_docs, q_len].
        Returns (dQ f64 [q_len, d], dD f64 shaped like D), None for an output not asked for."""
        Q, D = _c(Q), _c(D)
        n_docs, nd, off = self._layout(D, offsets)
        q_len, d = Q.shape
        ta = _c(tok_arg, np.int32).reshape(n_docs, q_len)
        g = _c(grad, np.float32).reshape(n_docs)
        dQ = np.empty((q_len, d), dtype=np.float64) if want_dQ else None
        dD = np.empty(D.shape, dtype=np.float64) if want_dD else None
        self._rc(self.lib.oracle_maxsim_backward(_ptr(Q), q_len, _ptr(D), _ptr(off), n_docs, nd, d,
                                                 DTYPES[dtype], _ptr(ta), _ptr(g), _ptr(dQ),
                                                 _ptr(dD)), "maxsim_backward")
        return dQ, dD

    def pq_tables(self, Q, dtype: str, C) -> np.ndarray:
        """T[i][m][k] (float64) for query Q [q_len, M*dsub] and codebook C [M, K, dsub]."""
        Q, C = _c(Q), _c(C, np.float32)
        M, K, dsub = C.shape
        T = np.empty((Q.shape[0], M, K), dtype=np.float64)
        self._rc(self.lib.oracle_pq_tables(_ptr(Q), Q.shape[0], DTYPES[dtype], _ptr(C), M, K, dsub,
                                           _ptr(T)), "pq_tables")
        return T

    def maxsim_pq(self, T, codes, offsets=None, nd=0, nthreads=None) -> np.ndarray:
        """PQ scoring with tables T [q_len, M, K] and codes [n_tokens, M] (CSR when offsets is
        given, else fixed docs of nd tokens)."""
        T, codes = _c(T, np.float64), _c(codes, np.uint8)
        q_len, M, K = T.shape
        off = _c(offsets, np.int64)
        n_docs = (len(off) - 1) if off is not None else codes.shape[0] // max(nd, 1)
        out = np.empty(n_docs, dtype=np.float64)
        self._rc(self.lib.oracle_maxsim_pq(_ptr(T), q_len, M, K, _ptr(codes), _ptr(off), n_docs,
                                           nd, _ptr(out), _threads(nthreads)), "maxsim_pq")
        return out


_default = None


def get() -> Oracle:
    """The oracle built from oracle/maxsim_oracle.c (compiled on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle(build(force=False))
    return _default


def maxsim_fixed(*a, **k):
    return get().maxsim_fixed(*a, **k)


def maxsim_csr(*a, **k):
    return get().maxsim_csr(*a, **k)


def maxsim_i8(*a, **k):
    return get().maxsim_i8(*a, **k)


def pq_tables(*a, **k):
    return get().pq_tables(*a, **k)


def maxsim_argmax(*a, **k):
    return get().maxsim_argmax(*a, **k)


def topk(scores, k: int):
    """The k best entries of each row of scores by (score descending, index ascending), the
    ordering used to rank documents (a library sort as the step). Returns (values [rows, k],
    indices [rows, k]); a row shorter than k is padded with -inf and index -1."""
    S = np.atleast_2d(np.asarray(scores))
    rows, n = S.shape
    vals = np.full((rows, k), -np.inf, dtype=S.dtype)
    idx = np.full((rows, k), -1, dtype=np.int64)
    for r in range(rows):
        order = np.lexsort((np.arange(n), -S[r]))[:k]
        vals[r, :len(order)] = S[r, order]
        idx[r, :len(order)] = order
    return vals, idx


def maxsim_batch(Qs, D, dtype: str, offsets=None, nthreads=None) -> np.ndarray:
    """Several queries Qs [n_q, q_len, d] against the same documents: by definition one
    single-query oracle score per (query, document); returns float64 [n_q, n_docs]."""
    if offsets is None:
        return np.stack([maxsim_fixed(q, D, dtype, nthreads=nthreads) for q in Qs])
    return np.stack([maxsim_csr(q, D, offsets, dtype, nthreads=nthreads) for q in Qs])


def maxsim_backward(*a, **k):
    return get().maxsim_backward(*a, **k)


def maxsim_pq(*a, **k):
    return get().maxsim_pq(*a, **k)


def score_corpus(c, nthreads=None) -> np.ndarray:
    """Oracle scores of a gen.Corpus (dense or INT8 storage)."""
    if c.dtype == "i8":
        return maxsim_i8(c.Q, c.q_scale, c.D, c.d_scale, c.offsets, nthreads)[0]
    if c.offsets is None:
        return maxsim_fixed(c.Q, c.D, c.dtype, nthreads=nthreads)
    return maxsim_csr(c.Q, c.D, c.offsets, c.dtype, nthreads=nthreads)
