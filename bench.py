#!/usr/bin/env python3
"""MaxSim scoring benchmark on one MI355X: docs/s and achieved bandwidth or throughput.

A step is one pass of the scoring path over the whole synthetic corpus, inputs
already resident in HBM. The default workload is the ColBERTv2 shape the pages
quote their headline on (TileMaxSim deep reading, section 4, Table 1): one query
of 32 tokens against 100,000 documents of 128 tokens, d=128, bf16.

Prints one JSON line. `roofline` covers the step's dominant kernel: algorithmic
bytes (memory-bound paths), FLOPs / integer ops (matrix-core-bound paths) or
table-lookup bytes (PQ) per launch, divided by its average duration measured with
HIP events recorded on the stream the kernel runs on. `cpu_baseline` times the
float64 oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks (dense): HBM3E 8 TB/s; MFMA bf16/fp16 2.5 PFLOP/s, int8 5.0 POP/s,
# fp32 157.3 TFLOP/s. LDS: 256 CUs x 128 B/clk x 2.4 GHz (derived, see the design notes).
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3, "i8": 5000.0}
# LDS: 256 CUs x 256 B per clock x 2.4 GHz. gfx950 serves 128-bit LDS reads at 256 B per clock
# per CU: maxsim_calib_lds measures 134 TB/s of contiguous ds_read_b128, above what 128 B per
# clock would allow (78.6 TB/s).
LDS_PEAK_GBS = 256 * 256 * 2.4
METRIC = "docs/s + % HBM peak, MaxSim B=100K Nq=32 Nd=128 d=128 bf16"

# layout: fixed (D [B, nd, d]) or csr (lognormal lengths, median 70, sigma 0.5, 8..512).
# path: dense (bf16/fp16/fp32), i8 (INT8 x INT8, per-token scales), pq (tables + lookups),
#       train (scores with argmax, then dQ and dD of sum_b g_b score_b in the input dtype),
#       batch (n_q queries of q_len tokens scored in one pass over the documents).
# pool: build the corpus from this many distinct seeded documents repeated to B.
_CB = dict(layout="fixed", path="dense", q_len=32, nd=128, d=128, dtype="bf16", seed=2)
WORKLOADS = {
    "colbert-b100k": dict(_CB, B=100_000),
    "colbert-b1k": dict(_CB, B=1_000),
    "colbert-b10k": dict(_CB, B=10_000),
    "colbert-b500k": dict(_CB, B=500_000, pool=50_000),
    "colbert-nd32": dict(_CB, B=100_000, nd=32),
    "colbert-nd64": dict(_CB, B=100_000, nd=64),
    "colbert-nd256": dict(_CB, B=100_000, nd=256),
    "colbert-nd512": dict(_CB, B=100_000, nd=512, pool=50_000),
    "colbert-fp16": dict(_CB, B=100_000, dtype="fp16"),
    "colbert-fp32": dict(_CB, B=100_000, dtype="fp32"),
    "dtile-d64": dict(_CB, B=100_000, d=64, seed=3),
    "dtile-d256": dict(_CB, B=100_000, d=256, seed=3),
    "dtile-d768": dict(_CB, B=100_000, d=768, seed=3, pool=25_000),
    "colpali-bf16-b1k": dict(_CB, B=1_000, q_len=1024, nd=1024, seed=4),
    "colpali-bf16-b10k": dict(_CB, B=10_000, q_len=1024, nd=1024, seed=4, pool=2_048),
    "colpali-bf16-b50k": dict(_CB, B=50_000, q_len=1024, nd=1024, seed=4, pool=2_048),
    "colpali-bf16-b175k": dict(_CB, B=175_000, q_len=1024, nd=1024, seed=4, pool=2_048),
    "colbert-i8-b100k": dict(_CB, B=100_000, dtype="i8", path="i8"),
    "colpali-i8-b1k": dict(_CB, B=1_000, q_len=1024, nd=1024, seed=4, dtype="i8", path="i8"),
    "colpali-i8-b10k": dict(_CB, B=10_000, q_len=1024, nd=1024, seed=4, dtype="i8", path="i8",
                            pool=2_048),
    "colpali-i8-b50k": dict(_CB, B=50_000, q_len=1024, nd=1024, seed=4, dtype="i8", path="i8",
                            pool=2_048),
    "colpali-i8-b175k": dict(_CB, B=175_000, q_len=1024, nd=1024, seed=4, dtype="i8", path="i8",
                             pool=2_048),
    "csr-bf16": dict(_CB, B=100_000, layout="csr", seed=5),
    "csr-pq": dict(_CB, B=100_000, layout="csr", seed=5, path="pq"),
    "fixed-pq": dict(_CB, B=100_000, seed=5, path="pq"),
    "colbert-topk100-b100k": dict(_CB, B=100_000, topk=100),
    "batch-colbert-q32-topk100-b100k": dict(_CB, B=100_000, n_q=32, path="batch", topk=100),
    "batch-colbert-q32-b100k": dict(_CB, B=100_000, n_q=32, path="batch"),
    "batch-colbert-q8-b100k": dict(_CB, B=100_000, n_q=8, path="batch"),
    "train-colbert-b100k": dict(_CB, B=100_000, path="train"),
    "train-csr": dict(_CB, B=100_000, layout="csr", seed=5, path="train"),
    "train-colpali-b10k": dict(_CB, B=10_000, q_len=1024, nd=1024, seed=4, pool=2_048,
                               path="train"),
}
DEFAULT = "colbert-b100k"
# sources each stored traffic reading depends on: the dense bf16 kernel (headline) and the
# backward's dD kernel (training step)
KERNEL_SOURCES = {
    "dense": ["device_common.hpp", "host_common.hpp", "dense_kernel.hpp", "dense_variants.hpp",
              "dense_dispatch.hpp", "dense_bf16.hip", "dense_i8.hip"],
    "train": ["device_common.hpp", "host_common.hpp", "dense_kernel.hpp", "backward_kernel.hpp",
              "backward.hip"],
    "dbatch": ["device_common.hpp", "host_common.hpp", "dense_kernel.hpp", "dense_dispatch.hpp",
               "dense_batch_kernel.hpp", "dense_batch.hip"],
    "tiled": ["device_common.hpp", "host_common.hpp", "dense_kernel.hpp", "tiled_kernel.hpp",
              "tiled_dispatch.hpp", "tiled_dense.hip", "tiled_i8.hip", "tiled_batch.hip"],
    "pq": ["device_common.hpp", "host_common.hpp", "dense_kernel.hpp", "pq_kernel.hpp"],
}


def short_query(w) -> bool:
    """Queries of up to 64 tokens go to the one-wave-per-document dense kernel (INT8 only at
    d = 64, 128 or 256); longer ones to the query-tiled kernel."""
    return w["q_len"] <= 64 and (w["dtype"] != "i8" or w["d"] in (64, 128, 256))


def dense_batch_fits(w) -> bool:
    """Up to 16 blocks of 16 query tokens (each query padded to whole blocks) with bf16 /
    fp16 rows of 128 or 256 bytes: the one-wave-per-document kernel with the queries in
    LDS."""
    row = w["d"] * esize(w["dtype"])
    blocks = w.get("n_q", 1) * -(-w["q_len"] // 16)
    return w["dtype"] in ("bf16", "fp16") and row in (128, 256) and blocks <= 16


def kernel_family(w) -> str:
    """Which kernel sources a workload's scoring runs: the one-wave-per-document dense
    kernel (short queries), the document-stationary kernel with the queries in LDS (up to
    16 query blocks), the query-tiled kernel (the rest), the PQ kernels, or the training
    step's backward."""
    if w["path"] in ("train", "pq"):
        return w["path"]
    if w["path"] != "batch" and short_query(w):
        return "dense"
    return "dbatch" if dense_batch_fits(w) else "tiled"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
PQ_M, PQ_K, PQ_DSUB = 16, 256, 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def boundary_events(n_steps: int, n_kernels: int, flush: bool):
    """Event indices of the timed steps: step i records events[i][k] before its kernel k and,
    where `closes[i]`, events[i][-1] after its last kernel. Without a cache flush between
    steps, the event that starts a step also ends the one before (events[i][-1] is
    events[i + 1][0]), so every kernel boundary costs one record. Returns (count, events,
    closes); every index in range(count) is recorded exactly once."""
    per = n_kernels + (1 if flush else 0)
    count = n_steps * per + (0 if flush else 1)
    events = [list(range(i * per, i * per + n_kernels + 1)) for i in range(n_steps)]
    closes = [flush or i == n_steps - 1 for i in range(n_steps)]
    return count, events, closes


class TimingEvent:
    """A HIP event for timing only, on the HIP runtime torch has loaded, created with
    hipEventDisableSystemFence. Recording a default event (torch.cuda.Event) performs a
    system-scope release, a write-back and invalidation of the caches, which costs several
    microseconds per record on MI355X and slows the work that follows; with the flag the
    record takes only its timestamp. The timed loop then runs as it would without events,
    and the event pairs still bracket each kernel on the stream it runs on. Read only after
    a device synchronisation."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            import torch
            torch.cuda.init()
            with open("/proc/self/maps") as f:
                paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
            if len(paths) != 1:
                raise RuntimeError(f"expected one loaded HIP runtime, found {sorted(paths)}")
            h = ctypes.CDLL(paths.pop())
            vp = ctypes.c_void_p
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            h.hipEventRecord.argtypes = [vp, vp]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            h.hipEventDestroy.argtypes = [vp]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream=None):
        import ctypes
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        rc = self._runtime().hipEventRecord(self._ev, ctypes.c_void_p(s.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "TimingEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = self._runtime().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        # events still alive at interpreter exit are left to the runtime's own teardown
        if self._hip is not None and self._ev and not sys.is_finalizing():
            self._hip.hipEventDestroy(self._ev)


def kernel_hash(path: str = "dense") -> str:
    """Hash of a kernel's sources and the compile flags, to tell whether stored counter
    readings still apply to the kernel that runs."""
    from maxsim_scoring_fwd_amd import build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(path, KERNEL_SOURCES["dense"]):
        h.update(open(os.path.join(ROOT, "maxsim_scoring_fwd_amd", "csrc", f), "rb").read())
    h.update(" ".join(build.HIP_FLAGS[:-2]).encode())  # flags without the include path
    return h.hexdigest()[:16]


def esize(dtype):
    return {"bf16": 2, "fp16": 2, "fp32": 4, "i8": 1}[dtype]


def intensity(w) -> float:
    """Matrix-core operations per byte of the document stream: 2 * n_q * q_len * d per token
    of d * element bytes (plus the fp32 scale of an INT8 token)."""
    row = w["d"] * esize(w["dtype"]) + (4 if w["dtype"] == "i8" else 0)
    return 2.0 * w.get("n_q", 1) * w["q_len"] * w["d"] / row


def bound_of(w):
    """The roofline that bounds the scoring kernel: HBM below the ridge point (peak
    operations per second over 8 TB/s), the matrix core above it; PQ lookups read LDS. A
    training step's bound is its longest launch's (train_roofline, once timed); before
    that, its dD kernel's, which writes a gradient row per token (HBM)."""
    if w["path"] == "train":
        return "hbm"
    if w["path"] == "pq":
        return "lds"
    ridge = MFMA_PEAK_TFLOPS[w["dtype"]] * 1e12 / (HBM_PEAK_GBS * 1e9)
    return "mfma" if intensity(w) > ridge else "hbm"


def _fill_rows(dst, seed, row0_of, nrows_total, d, dtype, device, chunk_rows, scale_dst=None):
    """Generate stream rows [0, nrows_total) in chunks into the device tensor dst (and scales)."""
    import torch

    import gen
    for r0 in range(0, nrows_total, chunk_rows):
        r1 = min(nrows_total, r0 + chunk_rows)
        if dtype == "i8":
            q, s = gen.tokens(seed, gen.S_DOCS, row0_of + r0, r1 - r0, d, "i8")
            dst[r0:r1] = torch.from_numpy(q).to(device)
            scale_dst[r0:r1] = torch.from_numpy(s).to(device)
        else:
            dst[r0:r1] = gen.to_device(gen.tokens(seed, gen.S_DOCS, row0_of + r0, r1 - r0, d, dtype),
                                       dtype, device)


def pq_codes(seed, n_tokens, C):
    """PQ codes of a corpus: the nearest-centroid codes of its generated unit-norm tokens
    (the document stream of the seed), encoded in chunks."""
    import numpy as np

    import gen
    out = np.empty((n_tokens, C.shape[0]), dtype=np.uint8)
    step = 1 << 20
    for r0 in range(0, n_tokens, step):
        r1 = min(n_tokens, r0 + step)
        out[r0:r1] = gen.encoded_codes(seed, gen.S_DOCS, r0, r1 - r0, C)
    return out


def make_inputs(w, device):
    """Generate the workload on the host in chunks and copy it to the device. With a pool,
    the first `pool` documents are generated and repeated (device copies) to fill B."""
    import numpy as np
    import torch

    import gen
    d, seed, dt = w["d"], w["seed"], w["dtype"]
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32,
           "i8": torch.int8}[dt]
    B = w["B"]
    inp = {}
    if dt == "i8":
        q, qs = gen.tokens(seed, gen.S_QUERY, 0, w["q_len"], d, "i8")
        inp["Q"] = torch.from_numpy(q).to(device)
        inp["q_scale"] = torch.from_numpy(qs).to(device)
    else:
        n_q = w.get("n_q", 1)
        q = gen.to_device(gen.tokens(seed, gen.S_QUERY, 0, n_q * w["q_len"], d, dt), dt, device)
        inp["Q"] = q.view(n_q, w["q_len"], d) if w["path"] == "batch" else q
    chunk_rows = max(1, (1 << 28) // (d * esize(dt)))

    if w["layout"] == "fixed":
        nd = w["nd"]
        pool = min(B, w.get("pool") or B)
        n_tok = B * nd
        inp["offsets"], inp["n_tokens"] = None, n_tok
        if w["path"] == "pq":
            C = gen.codebook(seed, PQ_M, PQ_K, PQ_DSUB)
            inp["C"] = torch.from_numpy(C).to(device)
            inp["codes"] = torch.from_numpy(pq_codes(seed, n_tok, C)).to(device)
            inp["T"] = torch.empty((w["q_len"], PQ_M, PQ_K), dtype=torch.float32, device=device)
            return inp
        D = torch.empty((B * nd, d), dtype=tdt, device=device)
        S = torch.empty(B * nd, dtype=torch.float32, device=device) if dt == "i8" else None
        _fill_rows(D, seed, 0, pool * nd, d, dt, device, chunk_rows, S)
        for b0 in range(pool, B, pool):
            b1 = min(B, b0 + pool)
            D[b0 * nd:b1 * nd] = D[0:(b1 - b0) * nd]
            if S is not None:
                S[b0 * nd:b1 * nd] = S[0:(b1 - b0) * nd]
        inp["D"] = D.view(B, nd, d)
        inp["d_scale"] = S
        if w["path"] == "train":
            _train_buffers(w, inp, device)
        return inp

    lens = gen.lengths(seed, B)
    off = gen.csr_offsets(lens)
    T = int(off[-1])
    inp["offsets"] = torch.from_numpy(off).to(device)
    inp["n_tokens"] = T
    if w["path"] == "pq":
        C = gen.codebook(seed, PQ_M, PQ_K, PQ_DSUB)
        inp["C"] = torch.from_numpy(C).to(device)
        inp["codes"] = torch.from_numpy(pq_codes(seed, T, C)).to(device)
        inp["T"] = torch.empty((w["q_len"], PQ_M, PQ_K), dtype=torch.float32, device=device)
        return inp
    D = torch.empty((T, d), dtype=tdt, device=device)
    S = torch.empty(T, dtype=torch.float32, device=device) if dt == "i8" else None
    _fill_rows(D, seed, 0, T, d, dt, device, chunk_rows, S)
    inp["D"], inp["d_scale"] = D, S
    if w["path"] == "train":
        _train_buffers(w, inp, device)
    return inp


def _train_buffers(w, inp, device):
    """Outputs of the training step: per-token maxima and argmax, an upstream gradient
    g_b ~ N(0, 1) per document (seeded), dQ and dD in the input dtype, the dQ workspace."""
    import numpy as np
    import torch

    import maxsim_scoring_fwd_amd as ms
    B, q, d = w["B"], w["q_len"], w["d"]
    inp["tok_max"] = torch.empty((B, q), dtype=torch.float32, device=device)
    inp["tok_arg"] = torch.empty((B, q), dtype=torch.int32, device=device)
    g = np.random.default_rng(w["seed"]).standard_normal(B).astype(np.float32)
    inp["grad"] = torch.from_numpy(g).to(device)
    inp["dQ"] = torch.empty((q, d), dtype=inp["D"].dtype, device=device)
    inp["dD"] = torch.empty(inp["D"].shape, dtype=inp["D"].dtype, device=device)
    inp["workspace"] = torch.empty(max(16, ms.backward_workspace_size(q, d, B)), dtype=torch.uint8,
                                   device=device)


def work_per_launch(w, inp):
    """Algorithmic work of the dominant kernel per launch: (amount, unit of the rate)."""
    n_tok, q, d, B = inp["n_tokens"], w["q_len"], w["d"], w["B"]
    bound = bound_of(w)
    if w["path"] == "train":
        return train_dd_bytes(w, inp), "GB/s"
    if bound == "hbm":
        n_q = w.get("n_q", 1)
        b = n_tok * d * esize(w["dtype"]) + n_q * (q * d * esize(w["dtype"]) + B * 4)
        if w["dtype"] == "i8":
            b += (n_tok + q) * 4  # fp32 scale per token
        if inp["offsets"] is not None:
            b += (B + 1) * 8
        return b, "GB/s"
    if bound == "mfma":
        return 2 * w.get("n_q", 1) * q * n_tok * d, ("TOP/s" if w["dtype"] == "i8" else "TFLOP/s")
    return n_tok * q * PQ_M * 4, "GB/s"  # fp32 table entries looked up


def train_dd_bytes(w, inp):
    """Algorithmic bytes of the dD kernel: every document token's gradient row written once
    (input dtype), the argmax and the upstream gradient read once, the query read once, the
    offsets of a CSR corpus."""
    n_tok, q, d, B, e = inp["n_tokens"], w["q_len"], w["d"], w["B"], esize(w["dtype"])
    b = n_tok * d * e + B * q * 4 + B * 4 + q * d * e
    if inp["offsets"] is not None:
        b += (B + 1) * 8
    return b


def train_roofline(w, inp, name):
    """Roofline of one launch of the training step, (bound, work per launch, unit, kernel
    family): the forward with per-token argmax by its intensity (the matrix core above the
    ridge, else the bytes it reads and writes: documents, query, scores, per-token maxima and
    argmax), dQ by the rows it gathers, dD by the rows it writes."""
    n_tok, q, d, B, e = inp["n_tokens"], w["q_len"], w["d"], w["B"], esize(w["dtype"])
    off = (B + 1) * 8 if inp["offsets"] is not None else 0
    if name == "maxsim_argmax":
        fam = "dense" if short_query(w) else "tiled"
        ridge = MFMA_PEAK_TFLOPS[w["dtype"]] * 1e12 / (HBM_PEAK_GBS * 1e9)
        if intensity(w) > ridge:
            return "mfma", 2 * q * n_tok * d, "TFLOP/s", fam
        return "hbm", n_tok * d * e + q * d * e + B * 4 + B * q * 8 + off, "GB/s", fam
    if name == "backward_dq":
        return "hbm", B * q * (d * e + 4) + B * 4 + q * d * e * 2, "GB/s", "train"
    return "hbm", train_dd_bytes(w, inp), "GB/s", "train"


def hbm_bytes(w, inp):
    """Bytes every document token costs in HBM (for context on mfma / lds-bound paths)."""
    if w["path"] == "pq":
        return inp["n_tokens"] * PQ_M + w["B"] * 4
    if w["path"] == "train":
        # forward: D read, scores + per-token maxima and argmax written; dQ: the chosen rows
        # gathered; dD: gradient rows written
        e, q, d, B = esize(w["dtype"]), w["q_len"], w["d"], w["B"]
        fwd = inp["n_tokens"] * d * e + B * 4 + B * q * 8
        return fwd + B * q * (d * e + 4) + train_dd_bytes(w, inp)
    b = inp["n_tokens"] * (w["d"] * esize(w["dtype"]) + (4 if w["dtype"] == "i8" else 0))
    return b + w.get("n_q", 1) * w["B"] * 4


def launches(ms, w, inp, out):
    """The kernel launches of one step, as (name, callable). The roofline is taken on the
    dominant one: the scoring kernel; in a training step the longest of its launches."""
    steps = _scoring_launches(ms, w, inp, out)
    if w.get("topk"):
        n_q = w.get("n_q", 1)
        scores = out.view(n_q, w["B"]) if n_q > 1 else out
        k = w["topk"]
        inp["topk_vals"] = torch_empty_like_rows(out, n_q, k, "float32")
        inp["topk_idx"] = torch_empty_like_rows(out, n_q, k, "int32")
        need = ms.topk_workspace_size(w["B"], n_q, k)
        inp["topk_ws"] = torch_empty_like_rows(out, 1, max(need, 16), "uint8")
        steps.append(("topk", lambda: ms.maxsim_topk(scores, k, out_scores=inp["topk_vals"],
                                                      out_index=inp["topk_idx"],
                                                      workspace=inp["topk_ws"])))
    return steps


def dominant_index(steps):
    names = [n for n, _ in steps]
    for n in ("maxsim", "maxsim_batch", "maxsim_i8", "pq_score"):
        if n in names:
            return names.index(n)
    return len(steps) - 1


def torch_empty_like_rows(ref, rows, k, dtype):
    import torch
    shape = (k,) if rows == 1 else (rows, k)
    return torch.empty(shape, dtype=getattr(torch, dtype), device=ref.device)


def _scoring_launches(ms, w, inp, out):
    """The scoring launches of one step (the whole step without top-k)."""
    if w["path"] == "batch":
        return [("maxsim_batch", lambda: ms.maxsim_score_batch(inp["Q"], inp["D"], inp["offsets"],
                                                              out=out.view(w["n_q"], w["B"])))]
    if w["path"] == "train":
        off, D = inp["offsets"], inp["D"]
        fwd = lambda: ms.maxsim_score_argmax(inp["Q"], D, off, out=out, tok_max=inp["tok_max"],
                                             tok_arg=inp["tok_arg"])
        bwd = lambda q, dd: ms.maxsim_backward(inp["Q"], D, inp["tok_arg"], inp["grad"], off,
                                               want_dQ=q, want_dD=dd, grad_dtype=D.dtype,
                                               dQ=inp["dQ"], dD=inp["dD"],
                                               workspace=inp["workspace"])
        # dD before dQ, the order maxsim_backward itself launches them in when asked for both
        # (dD right after the forward: 100K ColBERT documents 1.241 -> 1.212 ms per step,
        # ColPali 3.31-3.37 -> 3.19-3.21 ms)
        return [("maxsim_argmax", fwd), ("backward_dd", lambda: bwd(False, True)),
                ("backward_dq", lambda: bwd(True, False))]
    if w["path"] == "pq":
        steps = [("pq_tables", lambda: ms.maxsim_pq_tables(inp["Q"], inp["C"], T=inp["T"]))]
        if inp["offsets"] is None:
            steps.append(("pq_score", lambda: ms.maxsim_score_pq(inp["T"], inp["codes"], nd=w["nd"],
                                                                 out=out)))
        else:
            steps.append(("pq_score", lambda: ms.maxsim_score_pq(inp["T"], inp["codes"],
                                                                 inp["offsets"], out=out)))
        return steps
    if w["path"] == "i8":
        return [("maxsim_i8", lambda: ms.maxsim_score_i8(inp["Q"], inp["q_scale"], inp["D"],
                                                         inp["d_scale"], inp["offsets"], out=out))]
    if inp["offsets"] is None:
        return [("maxsim", lambda: ms.maxsim_score_fixed(inp["Q"], inp["D"], out=out))]
    return [("maxsim", lambda: ms.maxsim_score(inp["Q"], inp["D"], inp["offsets"], out=out))]


def cpu_baseline(w, budget_s: float):
    """Oracle on the host cores over the first documents of the same workload, sized to take
    about budget_s seconds."""
    import numpy as np

    import gen
    import oracle
    # every host core the process may use (its CPU affinity; OMP_NUM_THREADS where the
    # environment sets a smaller share)
    threads = oracle.host_threads()
    seed, d, dt, q = w["seed"], w["d"], w["dtype"], w["q_len"]

    def score(n):
        if w["layout"] == "fixed":
            off = None
            n_tok = n * w["nd"]
        else:
            off = gen.csr_offsets(gen.lengths(seed, w["B"])[:n])
            n_tok = int(off[-1])
        if w["path"] == "pq":
            Qh = gen.tokens(seed, gen.S_QUERY, 0, q, d, dt)
            C = gen.codebook(seed, PQ_M, PQ_K, PQ_DSUB)
            codes = pq_codes(seed, n_tok, C)
            t = time.perf_counter()
            T = oracle.pq_tables(Qh, dt, C)
            oracle.maxsim_pq(T, codes, offsets=off, nd=w.get("nd", 0), nthreads=threads)
            return time.perf_counter() - t
        if dt == "i8":
            Qh, qs = gen.tokens(seed, gen.S_QUERY, 0, q, d, "i8")
            Dh, ds = gen.tokens(seed, gen.S_DOCS, 0, n_tok, d, "i8")
            if off is None:
                Dh, ds = Dh.reshape(n, w["nd"], d), ds.reshape(n, w["nd"])
            t = time.perf_counter()
            oracle.maxsim_i8(Qh, qs, Dh, ds, off, nthreads=threads)
            return time.perf_counter() - t
        n_q = w.get("n_q", 1)
        Qh = gen.tokens(seed, gen.S_QUERY, 0, n_q * q, d, dt)
        Dh = gen.tokens(seed, gen.S_DOCS, 0, n_tok, d, dt)
        if off is None:
            Dh = Dh.reshape(n, w["nd"], d)
        if w["path"] == "batch":
            t = time.perf_counter()
            oracle.maxsim_batch(Qh.reshape(n_q, q, d), Dh, dt, offsets=off, nthreads=threads)
            return time.perf_counter() - t
        if w["path"] == "train":
            g = np.random.default_rng(seed).standard_normal(w["B"]).astype(np.float32)[:n]
            t = time.perf_counter()
            _, _, ta = oracle.maxsim_argmax(Qh, Dh, dt, offsets=off, nthreads=threads)
            oracle.maxsim_backward(Qh, Dh, dt, ta, g, offsets=off)
            return time.perf_counter() - t
        t = time.perf_counter()
        if off is None:
            oracle.maxsim_fixed(Qh, Dh, dt, nthreads=threads)
        else:
            oracle.maxsim_csr(Qh, Dh, off, dt, nthreads=threads)
        return time.perf_counter() - t

    n_q = w.get("n_q", 1)
    n0 = min(w["B"], 16 if q * n_q > 64 else 256)
    t0 = score(n0)
    n = int(min(w["B"], max(n0, n0 * budget_s / max(t0, 1e-6))))
    t = score(n) if n > n0 else t0
    unit = "docs/s" if n_q == 1 else "(query, document) scores/s"
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(n_q * n / t, 1), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"first {n} of the {w['B']} documents of the same workload "
                      f"(float64 oracle, {t:.1f} s)",
            "cpu_model": model, "host_cpus_visible": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


# Vector instructions per similarity in the query-tiled kernels' inner loops: INT8 a
# convert, the product with its scale product (the scale products themselves run on the
# matrix core) and half a three-way max; bf16 / fp16 half a three-way max.
VALU_PER_SIMILARITY = {"i8": 2.5, "bf16": 0.5, "fp16": 0.5}
# the forward with per-token argmax (bf16 / fp16): a compare and two selects per similarity
VALU_PER_SIMILARITY_ARGMAX = 3.0
# matrix-core cycles per 16 x 16 tile and query block relative to the dot products alone:
# INT8 adds a 32-cycle 16x16x1 4-block fp32 MFMA (scale products) per four 16-cycle int8
# ones at d = 128
MFMA_EXTRA = {"i8": 1.25, "bf16": 1.0, "fp16": 1.0}


def compute_ceilings(ms, w, achieved, stream, median_ms, valu_per_sim=None):
    """Measured ceilings of a matrix-core-bound workload, at the query-tiled kernels'
    occupancy (two waves per SIMD): the sustained MFMA rate of its dtype and the sustained
    vector-ALU rate, each alone, and two bounds for both together, from the workload's MFMA
    time T_M and vector time T_V at those rates:
      - no overlap: T_M + T_V (the rate if the two units only took turns);
      - measured overlap: max(T_M, T_V) + c * min(T_M, T_V), with c the share of the smaller
        time that maxsim_calib_mix leaves exposed when the two are balanced (V = 4 FMAs per
        int8 MFMA at two waves per SIMD: about as much vector time as matrix-core time).
        The calibration's units are independent streams; c is largest near balance, so
        this is the more demanding of the two bounds."""
    import torch
    sink = torch.zeros(65536, dtype=torch.float32, device="cuda")
    kind = 2 if w["dtype"] == "i8" else 0
    mfma_ops = ms.calib_mfma(kind, 4000, 2, sink)
    mfma = mfma_ops / (median_ms(lambda: ms.calib_mfma(kind, 4000, 2, sink)) * 1e-3) / 1e12
    valu_ops = ms.calib_valu(20000, 2, sink)
    valu = valu_ops / (median_ms(lambda: ms.calib_valu(20000, 2, sink)) * 1e-3) / 1e12
    # one VALU instruction per lane per FMA (2 FLOP): lane-instructions per second
    lane_instr = valu * 1e12 / 2
    ops_per_sim = 2 * w["d"]
    vps = valu_per_sim if valu_per_sim is not None else VALU_PER_SIMILARITY[w["dtype"]]
    valu_bound = lane_instr / vps * ops_per_sim / 1e12
    mfma_bound = mfma / MFMA_EXTRA[w["dtype"]]
    additive = 1.0 / (1.0 / mfma_bound + 1.0 / valu_bound)
    # exposed share of the smaller time in the balanced calibration: the launch's MFMA-only
    # time t0, its time with 4 FMAs per MFMA t4, and the vector time of those FMAs alone
    # (ops / 256 * V FLOP for V FMAs per MFMA)
    mix_ops = ms.calib_mix(0, 4000, 2, sink)
    t0 = median_ms(lambda: ms.calib_mix(0, 4000, 2, sink))
    t4 = median_ms(lambda: ms.calib_mix(4, 4000, 2, sink))
    tv4 = mix_ops / 256 * 4 / (valu * 1e12) * 1e3
    c = min(1.0, max(0.0, (t4 - max(t0, tv4)) / min(t0, tv4)))
    tm, tv = 1.0 / mfma_bound, 1.0 / valu_bound
    overlap = 1.0 / (max(tm, tv) + c * min(tm, tv))
    return {"mfma_sustained_TOPs_2w": round(mfma, 1),
            "frac_of_mfma_sustained": round(achieved / mfma, 4),
            "valu_fp32_TFLOPs_2w": round(valu, 1),
            "valu_per_similarity": vps,
            "valu_bound_TOPs": round(valu_bound, 1),
            "mfma_plus_valu_bound_TOPs": round(additive, 1),
            "frac_of_mfma_plus_valu_bound": round(achieved / additive, 4),
            "mix_exposed_share": round(c, 3),
            "mfma_valu_overlap_bound_TOPs": round(overlap, 1),
            "frac_of_mfma_valu_overlap_bound": round(achieved / overlap, 4)}


def lds_ceilings(ms, achieved, median_ms):
    """Measured LDS read rates: contiguous 128-bit reads, and the PQ lookup pattern (16-byte
    reads of random table rows) that bounds the PQ scoring kernel."""
    import torch
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    out = {}
    for pat, name in ((0, "contiguous"), (1, "pq_pattern")):
        b = ms.calib_lds(pat, 2000, sink)
        out[f"lds_read_GBps_{name}"] = round(b / (median_ms(lambda: ms.calib_lds(pat, 2000, sink))
                                                  * 1e-3) / 1e9, 1)
    out["frac_of_lds_pq_pattern"] = round(achieved / out["lds_read_GBps_pq_pattern"], 4)
    return out


def calib_suite():
    """The device's measured ceilings, one JSON line: stream read and write, sustained MFMA
    rates, the vector-ALU rate, the matrix core and vector ALU side by side, and LDS reads."""
    import torch

    import maxsim_scoring_fwd_amd as ms
    dev = torch.device("cuda:0")
    sink = torch.zeros(65536, dtype=torch.float32, device=dev)
    usink = torch.zeros(65536, dtype=torch.int32, device=dev)

    def med(fn, reps=7):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = TimingEvent(), TimingEvent()
            a.record()
            r = fn()
            b.record()
            torch.cuda.synchronize()
            ts.append((a.elapsed_time(b), r))
        ts.sort(key=lambda x: x[0])
        return ts[len(ts) // 2]

    out = {"device": torch.cuda.get_device_name(0)}
    buf = torch.ones(1 << 30, dtype=torch.int32, device=dev)
    # one workgroup of 4 waves per CU, and as many as fit: the faster is the ceiling
    for n, key in ((1, "stream_read_1wg_per_cu_GBps"), (0, "stream_read_full_occupancy_GBps")):
        t, _ = med(lambda: ms.calib_read(buf, usink, wgs_per_cu=n))
        out[key] = round(buf.numel() * 4 / (t * 1e-3) / 1e9, 1)
    out["stream_read_GBps"] = max(out["stream_read_1wg_per_cu_GBps"],
                                  out["stream_read_full_occupancy_GBps"])
    # contiguous ranges at two workgroups per CU, and blocks in turn at one: the faster is
    # the ceiling
    for n, c, key in ((2, True, "stream_write_contig_2wg_per_cu_GBps"),
                      (1, False, "stream_write_blocks_1wg_per_cu_GBps")):
        t, _ = med(lambda: ms.calib_write(buf, wgs_per_cu=n, contig=c))
        out[key] = round(buf.numel() * 4 / (t * 1e-3) / 1e9, 1)
    out["stream_write_GBps"] = max(out["stream_write_contig_2wg_per_cu_GBps"],
                                   out["stream_write_blocks_1wg_per_cu_GBps"])
    del buf
    for kind, name in ((0, "bf16_16x16x32"), (1, "bf16_32x32x16"), (2, "i8_16x16x64"), (3, "i8_32x32x32")):
        for w in (2, 4):
            t, ops = med(lambda: ms.calib_mfma(kind, 4000, w, sink))
            out[f"mfma_{name}_w{w}_TOPs"] = round(ops / (t * 1e-3) / 1e12, 1)
    for w in (1, 2, 4, 8):
        t, ops = med(lambda: ms.calib_valu(20000, w, sink))
        out[f"valu_fp32_fma_w{w}_TFLOPs"] = round(ops / (t * 1e-3) / 1e12, 1)
    for w in (2, 4):
        for v in (0, 1, 2, 4, 8):
            t, ops = med(lambda: ms.calib_mix(v, 4000, w, sink))
            out[f"mix_w{w}_v{v}_ms"] = round(t, 4)
    for pat, name in ((0, "contiguous"), (1, "pq_pattern")):
        t, b = med(lambda: ms.calib_lds(pat, 2000, usink))
        out[f"lds_read_{name}_GBps"] = round(b / (t * 1e-3) / 1e9, 1)
    print(json.dumps(out), flush=True)


def copy_probe(mib: int, steps: int):
    """Run the plain 128-bit copy kernel on a buffer of known size (counter calibration)."""
    import torch

    import maxsim_scoring_fwd_amd as ms
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        ms.calib_copy(src, dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "launches": steps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 skips it)")
    ap.add_argument("--no-calib", action="store_true", help="skip the stream-read calibration")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run the copy kernel on this many MiB, --steps times")
    ap.add_argument("--calib-suite", action="store_true",
                    help="only measure the device's ceilings (calibration kernels), one JSON line")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the scoring path runs on a single MI355X and "
              "shards across GPUs by documents with no exchange; run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, args.steps)
        return
    if args.calib_suite:
        calib_suite()
        return

    import torch

    import maxsim_scoring_fwd_amd as ms
    ms.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    log(f"workload {args.workload}: {w}")
    t = time.perf_counter()
    inp = make_inputs(w, dev)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({time.perf_counter() - t:.1f} s)")
    n_q = w.get("n_q", 1)  # scores per document: one per query
    out = torch.empty(n_q * w["B"], dtype=torch.float32, device=dev)
    steps_fns = launches(ms, w, inp, out)
    work, rate_unit = work_per_launch(w, inp)

    # The MI355X L2 + Infinity Cache hold ~288 MiB: smaller corpora are flushed between
    # steps and their throughput is taken from the kernel events alone.
    footprint = hbm_bytes(w, inp)
    flush = footprint < (1 << 30)
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev) if flush else None

    def one_step(evs=None, close=True):
        for k, (_, fn) in enumerate(steps_fns):
            if evs is not None:
                evs[k].record(stream)
            fn()
        if evs is not None and close:
            evs[-1].record(stream)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        one_step()
        if flush:
            scratch.zero_()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    nk = len(steps_fns)
    # one event at every kernel boundary of the timed steps (boundary_events)
    n_ev, ev_idx, closes = boundary_events(args.steps, nk, flush)
    pool = [TimingEvent() for _ in range(n_ev)]
    evs = [[pool[j] for j in idx] for idx in ev_idx]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(evs[i], close=closes[i])
        if flush:
            scratch.zero_()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [e[0].elapsed_time(e[-1]) for e in evs]
    per_launch = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / len(evs)
                  for j in range(len(steps_fns))]
    family = kernel_family(w)
    bound = bound_of(w)
    if w["path"] == "train":
        # the training step's launches differ by shape: the longest one is the dominant kernel
        di = max(range(len(steps_fns)), key=lambda j: per_launch[j])
        bound, work, rate_unit, family = train_roofline(w, inp, steps_fns[di][0])
    else:
        di = dominant_index(steps_fns)
    dom_ms = [e[di].elapsed_time(e[di + 1]) for e in evs]  # the dominant kernel
    avg_step, avg_dom = sum(step_ms) / len(step_ms), sum(dom_ms) / len(dom_ms)
    log(f"timed {args.steps} steps: wall {wall * 1e3 / args.steps:.4f} ms/step, step events avg "
        f"{avg_step:.4f} ms, dominant kernel avg {avg_dom:.4f} ms, min {min(dom_ms):.4f} ms")

    if flush:
        value, ms_per_step = n_q * w["B"] / (avg_step * 1e-3), avg_step
    else:
        value, ms_per_step = n_q * w["B"] * args.steps / wall, wall * 1e3 / args.steps

    if bound == "mfma":
        achieved = work / (avg_dom * 1e-3) / 1e12
        peak = MFMA_PEAK_TFLOPS[w["dtype"]]
    else:
        achieved = work / (avg_dom * 1e-3) / 1e9
        peak = HBM_PEAK_GBS if bound == "hbm" else LDS_PEAK_GBS

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE)).get(args.workload)
        # a reading applies to the kernel family it was taken on (a training step's reading
        # is of its dD kernel, hashed as the backward's family)
        if rec and rec.get("kernel_hash") == kernel_hash(family):
            traffic = rec.get("bytes_per_launch")

    context = {"dominant_kernel": steps_fns[di][0], "kernel_ms_avg": round(avg_dom, 5),
               "kernel_ms_min": round(min(dom_ms), 5), "work_per_launch": work,
               "hbm_bytes_per_step": footprint,
               "hbm_GBps": round(footprint / (avg_step * 1e-3) / 1e9, 1),
               "caches_flushed_between_steps": flush, "kernel_hash": kernel_hash(family)}
    if len(steps_fns) > 1:
        context["kernel_ms_per_launch"] = {n: round(per_launch[j], 5)
                                           for j, (n, _) in enumerate(steps_fns)}
    if w.get("pool") and w["pool"] < w["B"]:
        context["pool"] = f"{w['pool']} distinct documents repeated to {w['B']}"
    if not args.no_calib:
        buf = torch.empty(1 << 30, dtype=torch.int32, device=dev)  # 4 GiB
        buf.fill_(1)
        sink = torch.zeros(65536, dtype=torch.int32, device=dev)
        def median_ms(fn):
            for _ in range(3):
                fn()
            cs = [TimingEvent() for _ in range(10)]
            ce = [TimingEvent() for _ in range(10)]
            for i in range(10):
                cs[i].record(stream)
                fn()
                ce[i].record(stream)
            torch.cuda.synchronize()
            return sorted(s.elapsed_time(e) for s, e in zip(cs, ce))[5]

        # the stream read with one workgroup of 4 waves per CU and with as many as fit: the
        # faster of the two is the ceiling
        reads = {n: buf.numel() * 4 / (median_ms(lambda: ms.calib_read(buf, sink, wgs_per_cu=n))
                                       * 1e-3) / 1e9 for n in (1, 0)}
        stream_gbs = max(reads.values())
        context["stream_read_GBps"] = round(stream_gbs, 1)
        context["stream_read_GBps_by_launch"] = {"1_wg_per_cu": round(reads[1], 1),
                                                 "full_occupancy": round(reads[0], 1)}
        if flush and bound == "hbm" and w["path"] != "train":
            # a corpus this small is dominated by launch and ramp-up: the same stream read
            # over the same number of bytes, caches flushed the same way, is its ceiling
            n_small = min(footprint // 16 * 4, buf.numel())
            small = buf[:n_small]
            small_gbs = 0.0
            for n in (1, 0):  # the faster of the two launch shapes, as above
                ts = []
                for i in range(13):
                    scratch.zero_()
                    cs, ce = TimingEvent(), TimingEvent()
                    cs.record(stream)
                    ms.calib_read(small, sink, wgs_per_cu=n)
                    ce.record(stream)
                    torch.cuda.synchronize()
                    if i >= 3:
                        ts.append(cs.elapsed_time(ce))
                small_gbs = max(small_gbs, n_small * 4 / (sorted(ts)[len(ts) // 2] * 1e-3) / 1e9)
            context["stream_read_same_bytes_GBps"] = round(small_gbs, 1)
            context["frac_of_stream_read_same_bytes"] = round(achieved / small_gbs, 4)
            log(f"stream read of the same {n_small * 4} bytes, caches flushed: {small_gbs:.0f} GB/s")
        if bound == "mfma" and w["dtype"] != "fp32" and w["path"] != "train":
            context.update(compute_ceilings(ms, w, achieved, stream, median_ms))
        if bound == "lds":
            context.update(lds_ceilings(ms, achieved, median_ms))
        if bound == "mfma" and w["path"] == "train":
            context.update(compute_ceilings(ms, w, achieved, stream, median_ms,
                                            valu_per_sim=VALU_PER_SIMILARITY_ARGMAX))
        elif w["path"] == "train" and steps_fns[di][0] == "backward_dd":
            # the dD kernel mostly writes: its ceiling is the streaming-write rate
            # the faster of two launch shapes of the stream write
            wr_gbs = max(buf.numel() * 4 / (median_ms(lambda: ms.calib_write(
                buf, wgs_per_cu=n, contig=c)) * 1e-3) / 1e9 for n, c in ((2, True), (1, False)))
            context["stream_write_GBps"] = round(wr_gbs, 1)
            context["frac_of_stream_write"] = round(achieved / wr_gbs, 4)
            log(f"stream-write ceiling {wr_gbs:.0f} GB/s")
        elif bound == "hbm":
            context["frac_of_stream_read"] = round(achieved / stream_gbs, 4)
        del buf
        log(f"stream-read ceiling {stream_gbs:.0f} GB/s")
    if bound == "hbm" and w["path"] != "train" and intensity(w) > 64:
        # close to the ridge: the matrix-core rate beside the HBM rate
        mfma_tops = 2 * n_q * w["q_len"] * inp["n_tokens"] * w["d"] / (avg_dom * 1e-3) / 1e12
        context["mfma_TOPs"] = round(mfma_tops, 1)
        context["frac_of_mfma_peak"] = round(mfma_tops / MFMA_PEAK_TFLOPS[w["dtype"]], 4)

    cpu = None
    if args.cpu_budget > 0:
        log("timing the CPU oracle baseline ...")
        cpu = cpu_baseline(w, args.cpu_budget)
        log(f"cpu baseline {cpu}")

    cfg = {"workload": args.workload, "layout": w["layout"], "path": w["path"], "n_docs": w["B"],
           "q_len": w["q_len"], "d": w["d"], "storage": w["dtype"]}
    if w["layout"] == "fixed":
        cfg["nd"] = w["nd"]
    else:
        cfg["n_tokens"] = inp["n_tokens"]
        cfg["lengths"] = "lognormal median 70 sigma 0.5 clipped 8..512"
    if w["path"] == "pq":
        cfg["pq"] = {"M": PQ_M, "K": PQ_K, "dsub": PQ_DSUB}
    if n_q > 1:
        cfg["n_q"] = n_q
    if w.get("topk"):
        cfg["topk"] = w["topk"]
    if w["path"] == "train":
        cfg["step"] = ("scores with per-token argmax, then dQ and dD of sum_b g_b score_b "
                       f"(g_b ~ N(0,1), gradients in {w['dtype']})")
    line = {
        "metric": METRIC if args.workload == DEFAULT else
        (f"docs/s, MaxSim {args.workload}" if n_q == 1 else f"scores/s, MaxSim {args.workload}"),
        "value": round(value, 1),
        "unit": "docs/s" if n_q == 1 else "(query, document) scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"i8": "int8", "fp32": "fp32"}.get(w["dtype"], w["dtype"]),
        "data": "synthetic (seeded unit-norm Gaussian token embeddings)",
        "config": cfg,
        "roofline": {"bound": bound, "achieved": round(achieved, 1), "peak": peak,
                     "unit": rate_unit, "frac": round(achieved / peak, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "context": context,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
