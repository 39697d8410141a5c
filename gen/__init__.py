"""Seeded synthetic inputs for MaxSim scoring (shared by the oracle side and the GPU side).

This module produces inputs only and holds none of the scoring arithmetic. The
random numbers are counter-based (SplitMix64 + Box-Muller, see maxsim_gen.c),
so any document can be regenerated on its own and results do not depend on the
thread count.

Storage formats returned (numpy):
  bf16 -> uint16 raw bits, fp16 -> float16, fp32 -> float32,
  i8   -> int8 tokens plus a float32 per-token scale.

Streams of one seed: query 0, docs 1, planting 2, lengths 3, codebook 4,
noise 5, codes 6.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "maxsim_gen.c")
_SO = os.path.join(_HERE, "_maxsim_gen.so")

S_QUERY, S_DOCS, S_PLANT, S_LENGTHS, S_CODEBOOK, S_NOISE, S_CODES = range(7)
DTYPES = {"bf16": 0, "fp16": 1, "fp32": 2, "f64": 3, "i8": 4}
NP_STORAGE = {"bf16": np.uint16, "fp16": np.float16, "fp32": np.float32, "f64": np.float64,
              "i8": np.int8}


def build(force: bool = True) -> str:
    """Compile the generator shared library in place (gcc, no GPU code)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _SO)
    return _SO


_lib_cache = None


def _lib():
    global _lib_cache
    if _lib_cache is None:
        build(force=False)
        lib = ctypes.CDLL(_SO)
        u64, i64, i32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.gen_key.argtypes = [u64, u64]
        lib.gen_key.restype = u64
        lib.gen_u64.argtypes = [u64, u64]
        lib.gen_u64.restype = u64
        lib.gen_normal.argtypes = [u64, u64]
        lib.gen_normal.restype = ctypes.c_double
        lib.gen_unit_token.argtypes = [u64, u64, i64, i32, vp]
        lib.gen_tokens.argtypes = [u64, u64, i64, i64, i32, i32, vp, vp, i32]
        lib.gen_lengths.argtypes = [u64, u64, i64, ctypes.c_double, ctypes.c_double, i32, i32, vp]
        lib.gen_distinct.argtypes = [u64, u64, u64, i32, i64, vp]
        lib.gen_plant_doc.argtypes = [u64, u64, i64, i32, u64, u64, i64, i32, i32,
                                      ctypes.c_double, i32, vp, vp]
        lib.gen_codebook.argtypes = [u64, u64, i32, i32, i32, vp]
        lib.gen_codes.argtypes = [u64, u64, i64, i64, i32, i32, vp]
        lib.gen_pq_encode.argtypes = [vp, i64, i32, i32, i32, vp, vp]
        lib.gen_encoded_codes.argtypes = [u64, u64, i64, i64, i32, i32, i32, vp, vp, i32]
        lib.gen_round_f32_to_bf16.argtypes = [vp, i64, vp]
        lib.gen_round_f32_to_f16.argtypes = [vp, i64, vp]
        _lib_cache = lib
    return _lib_cache


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def default_threads() -> int:
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


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"gen: {what} rejected its arguments (rc={rc})")


def tokens(seed: int, stream: int, row0: int, nrows: int, d: int, dtype: str,
           nthreads: int | None = None):
    """Unit-norm Gaussian token rows [row0, row0+nrows) of a stream, stored as dtype.

    Returns the storage array [nrows, d]; for 'i8' returns (int8 array, float32 scales).
    """
    out = np.empty((nrows, d), dtype=NP_STORAGE[dtype])
    scale = np.empty(nrows, dtype=np.float32) if dtype == "i8" else None
    _check(_lib().gen_tokens(seed, stream, row0, nrows, d, DTYPES[dtype], _ptr(out), _ptr(scale),
                             nthreads or default_threads()), "gen_tokens")
    return (out, scale) if dtype == "i8" else out


def lengths(seed: int, n_docs: int, median: float = 70.0, sigma: float = 0.5, lo: int = 8,
            hi: int = 512) -> np.ndarray:
    out = np.empty(n_docs, dtype=np.int32)
    _check(_lib().gen_lengths(seed, S_LENGTHS, n_docs, median, sigma, lo, hi, _ptr(out)),
           "gen_lengths")
    return out


def distinct(seed: int, stream: int, salt: int, n: int, rng: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int64)
    _check(_lib().gen_distinct(seed, stream, salt, n, rng, _ptr(out)), "gen_distinct")
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _lib().gen_round_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def round_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _lib().gen_round_f32_to_f16(_ptr(x), x.size, _ptr(out))
    return out.view(np.float16)


def unit_token_f64(seed: int, stream: int, row: int, d: int) -> np.ndarray:
    x = np.empty(d, dtype=np.float64)
    _lib().gen_unit_token(seed, stream, row, d, _ptr(x))
    return x


@dataclass
class Corpus:
    """One query and a corpus of documents, in storage formats.

    Fixed layout: D is [n_docs, nd, d] and offsets is None.
    CSR layout:   D is [n_tokens, d] and offsets is int64 [n_docs + 1].
    For 'i8', q_scale / d_scale hold the per-token fp32 scales.
    """
    seed: int
    dtype: str
    d: int
    Q: np.ndarray
    D: np.ndarray
    n_docs: int
    nd: int = 0
    offsets: np.ndarray | None = None
    q_scale: np.ndarray | None = None
    d_scale: np.ndarray | None = None
    planted: np.ndarray = field(default_factory=lambda: np.zeros(0, dtype=np.int64))

    @property
    def q_len(self) -> int:
        return self.Q.shape[0]

    def doc_len(self, b: int) -> int:
        if self.offsets is None:
            return self.nd
        return int(self.offsets[b + 1] - self.offsets[b])


def _plant(c: Corpus, n_plant: int, sigma: float, q_row0: int = 0):
    """Plant n_plant near-duplicates of the query (distinct doc ids from the planting stream)."""
    if n_plant <= 0:
        return
    ids = distinct(c.seed, S_PLANT, 0, n_plant, c.n_docs)
    lib = _lib()
    for b in ids:
        b = int(b)
        L = c.doc_len(b)
        if c.offsets is None:
            rows = c.D[b]
            sc = None if c.d_scale is None else c.d_scale[b]
        else:
            s0 = int(c.offsets[b])
            rows = c.D[s0:s0 + L]
            sc = None if c.d_scale is None else c.d_scale[s0:s0 + L]
        rows_c = np.ascontiguousarray(rows)
        sc_c = None if sc is None else np.ascontiguousarray(sc)
        _check(lib.gen_plant_doc(c.seed, S_QUERY, q_row0, c.q_len, S_PLANT, S_NOISE, b, L, c.d,
                                 sigma, DTYPES[c.dtype], _ptr(rows_c), _ptr(sc_c)), "gen_plant_doc")
        rows[...] = rows_c
        if sc is not None:
            sc[...] = sc_c
    c.planted = ids


def fixed_corpus(seed: int, n_docs: int, q_len: int, nd: int, d: int, dtype: str = "bf16",
                 n_plant: int = 0, plant_sigma: float = 0.05,
                 nthreads: int | None = None) -> Corpus:
    """Fixed-length documents [n_docs, nd, d]; doc b token j is docs-stream row b*nd + j."""
    if dtype == "i8":
        Q, qs = tokens(seed, S_QUERY, 0, q_len, d, "i8", nthreads)
        D, ds = tokens(seed, S_DOCS, 0, n_docs * nd, d, "i8", nthreads)
        c = Corpus(seed, dtype, d, Q, D.reshape(n_docs, nd, d), n_docs, nd=nd, q_scale=qs,
                   d_scale=ds.reshape(n_docs, nd))
    else:
        Q = tokens(seed, S_QUERY, 0, q_len, d, dtype, nthreads)
        D = tokens(seed, S_DOCS, 0, n_docs * nd, d, dtype, nthreads).reshape(n_docs, nd, d)
        c = Corpus(seed, dtype, d, Q, D, n_docs, nd=nd)
    _plant(c, n_plant, plant_sigma)
    return c


def csr_offsets(lens: np.ndarray) -> np.ndarray:
    off = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=off[1:])
    return off


def csr_corpus(seed: int, n_docs: int, q_len: int, d: int, dtype: str = "bf16",
               lens: np.ndarray | None = None, median: float = 70.0, sigma: float = 0.5,
               lo: int = 8, hi: int = 512, n_plant: int = 0, plant_sigma: float = 0.05,
               nthreads: int | None = None) -> Corpus:
    """Variable-length documents stored CSR: D [n_tokens, d], offsets int64 [n_docs+1].

    Lengths are lognormal (median, sigma) clipped to [lo, hi] unless given. Token t of the
    corpus is docs-stream row t.
    """
    if lens is None:
        lens = lengths(seed, n_docs, median, sigma, lo, hi)
    off = csr_offsets(np.asarray(lens, dtype=np.int64))
    T = int(off[-1])
    if dtype == "i8":
        Q, qs = tokens(seed, S_QUERY, 0, q_len, d, "i8", nthreads)
        D, ds = tokens(seed, S_DOCS, 0, T, d, "i8", nthreads)
        c = Corpus(seed, dtype, d, Q, D, n_docs, offsets=off, q_scale=qs, d_scale=ds)
    else:
        Q = tokens(seed, S_QUERY, 0, q_len, d, dtype, nthreads)
        D = tokens(seed, S_DOCS, 0, T, d, dtype, nthreads)
        c = Corpus(seed, dtype, d, Q, D, n_docs, offsets=off)
    _plant(c, n_plant, plant_sigma)
    return c


def fixed_docs_subset(seed: int, doc_ids, nd: int, d: int, dtype: str,
                      n_plant_ids: np.ndarray | None = None, q_len: int = 0,
                      plant_sigma: float = 0.05):
    """Regenerate only the listed documents of a fixed corpus (for sampled checks).

    Returns storage [len(doc_ids), nd, d] (and scales for 'i8'), with the same planting as
    fixed_corpus applied to any listed doc that is in n_plant_ids.
    """
    ids = [int(b) for b in doc_ids]
    outs, scs = [], []
    for b in ids:
        r = tokens(seed, S_DOCS, b * nd, nd, d, dtype, 1)
        if dtype == "i8":
            outs.append(r[0])
            scs.append(r[1])
        else:
            outs.append(r)
    D = np.stack(outs) if outs else np.zeros((0, nd, d), dtype=NP_STORAGE[dtype])
    S = np.stack(scs) if scs else None
    if n_plant_ids is not None and len(n_plant_ids):
        pset = set(int(x) for x in n_plant_ids)
        lib = _lib()
        for k, b in enumerate(ids):
            if b in pset:
                rows = np.ascontiguousarray(D[k])
                sc = None if S is None else np.ascontiguousarray(S[k])
                _check(lib.gen_plant_doc(seed, S_QUERY, 0, q_len, S_PLANT, S_NOISE, b, nd, d,
                                         plant_sigma, DTYPES[dtype], _ptr(rows), _ptr(sc)),
                       "gen_plant_doc")
                D[k] = rows
                if S is not None:
                    S[k] = sc
    return (D, S) if dtype == "i8" else D


def codebook(seed: int, M: int = 16, K: int = 256, dsub: int = 8) -> np.ndarray:
    C = np.empty((M, K, dsub), dtype=np.float32)
    _check(_lib().gen_codebook(seed, S_CODEBOOK, M, K, dsub, _ptr(C)), "gen_codebook")
    return C


def codes(seed: int, n_tokens: int, M: int = 16, K: int = 256, row0: int = 0) -> np.ndarray:
    out = np.empty((n_tokens, M), dtype=np.uint8)
    _check(_lib().gen_codes(seed, S_CODES, row0, n_tokens, M, K, _ptr(out)), "gen_codes")
    return out


def pq_encode(x: np.ndarray, C: np.ndarray) -> np.ndarray:
    """Nearest-centroid PQ codes of double token rows x [n, M*dsub] (ties to the lowest k)."""
    M, K, dsub = C.shape
    x = np.ascontiguousarray(x, dtype=np.float64)
    C = np.ascontiguousarray(C, dtype=np.float32)
    out = np.empty((x.shape[0], M), dtype=np.uint8)
    _check(_lib().gen_pq_encode(_ptr(x), x.shape[0], M, K, dsub, _ptr(C), _ptr(out)),
           "gen_pq_encode")
    return out


def encoded_codes(seed: int, stream: int, row0: int, n: int, C: np.ndarray,
                  nthreads: int | None = None) -> np.ndarray:
    """Nearest-centroid PQ codes [n, M] of token rows [row0, row0 + n) of a stream, each
    generated in double and encoded as pq_encode does, without holding the vectors."""
    M, K, dsub = C.shape
    C = np.ascontiguousarray(C, dtype=np.float32)
    out = np.empty((n, M), dtype=np.uint8)
    _check(_lib().gen_encoded_codes(seed, stream, row0, n, M, K, dsub, _ptr(C), _ptr(out),
                                    nthreads or default_threads()), "gen_encoded_codes")
    return out


def tokens_f64(seed: int, stream: int, row0: int, nrows: int, d: int) -> np.ndarray:
    return tokens(seed, stream, row0, nrows, d, "f64")


# ---- the five workload shapes ----
# C1: 1 query (Nq=32) x 1000 docs (Nd=128), d=128, bf16, 10 planted near-duplicates, seed 1.
# C2: Nq=32, Nd=128, d=128, B in {1K, 10K, 100K, 500K}; Nd in {32, 64, 256, 512}; bf16/fp16/fp32.
# C3: Nq=32, Nd=128, B=100K, d in {64, 256, 768}, bf16.
# C4: Lq=Ld=1024, d=128, B in {1K, 10K, 50K, 175K}, bf16 and INT8 with per-token scales.
# C5: B=100K, lognormal lengths (median 70, clipped 8-512), CSR, Nq=32, d=128, bf16 or PQ codes
#     (M=16 subspaces of 8 dims, K=256 unit-norm Gaussian centroids).
SEEDS = {"C1": 1, "C2": 2, "C3": 3, "C4": 4, "C5": 5}


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Copy a storage array to a torch device tensor of the matching torch dtype
    (bf16 raw bits are reinterpreted as torch.bfloat16)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)
