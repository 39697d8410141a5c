#!/usr/bin/env python3
"""MaxSim scoring benchmark on one MI355X: docs/s and achieved HBM bandwidth.

A step is one call of the scoring path over the whole synthetic corpus, inputs
already resident in HBM. The default workload is the ColBERTv2 shape the pages
quote their headline on (TileMaxSim deep reading, section 4, Table 1): one query
of 32 tokens against 100,000 documents of 128 tokens, d=128, bf16.

Prints one JSON line. `roofline` covers the scoring kernel: algorithmic bytes per
launch divided by its average duration, measured with HIP events recorded on the
stream the kernel runs on. `cpu_baseline` times the float64 oracle on a bounded
sample of the same workload on the host cores.
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak
METRIC = "docs/s + % HBM peak, MaxSim B=100K Nq=32 Nd=128 d=128 bf16"

# name -> workload. kind: fixed (D [B, nd, d]) or csr (lognormal lengths, median 70, 8..512)
WORKLOADS = {
    "colbert-b100k": dict(kind="fixed", B=100_000, q_len=32, nd=128, d=128, dtype="bf16", seed=2),
    "colbert-b1k": dict(kind="fixed", B=1_000, q_len=32, nd=128, d=128, dtype="bf16", seed=2),
    "colbert-b10k": dict(kind="fixed", B=10_000, q_len=32, nd=128, d=128, dtype="bf16", seed=2),
    "colbert-b500k": dict(kind="fixed", B=500_000, q_len=32, nd=128, d=128, dtype="bf16", seed=2),
    "colbert-nd32": dict(kind="fixed", B=100_000, q_len=32, nd=32, d=128, dtype="bf16", seed=2),
    "colbert-nd64": dict(kind="fixed", B=100_000, q_len=32, nd=64, d=128, dtype="bf16", seed=2),
    "colbert-nd256": dict(kind="fixed", B=100_000, q_len=32, nd=256, d=128, dtype="bf16", seed=2),
    "colbert-nd512": dict(kind="fixed", B=100_000, q_len=32, nd=512, d=128, dtype="bf16", seed=2),
    "colbert-fp16": dict(kind="fixed", B=100_000, q_len=32, nd=128, d=128, dtype="fp16", seed=2),
    "colbert-fp32": dict(kind="fixed", B=100_000, q_len=32, nd=128, d=128, dtype="fp32", seed=2),
    "dtile-d64": dict(kind="fixed", B=100_000, q_len=32, nd=128, d=64, dtype="bf16", seed=3),
    "dtile-d256": dict(kind="fixed", B=100_000, q_len=32, nd=128, d=256, dtype="bf16", seed=3),
    "dtile-d768": dict(kind="fixed", B=100_000, q_len=32, nd=128, d=768, dtype="bf16", seed=3),
    "csr-bf16": dict(kind="csr", B=100_000, q_len=32, d=128, dtype="bf16", seed=5),
}
DEFAULT = "colbert-b100k"
KERNEL_SOURCES = ["device_common.hpp", "dense_kernel.hpp", "dense_variants.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "maxsim_scoring_fwd_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def esize(dtype):
    return 4 if dtype == "fp32" else 2


def make_inputs(w, device):
    """Generate the corpus on the host in chunks and copy it to the device."""
    import numpy as np
    import torch

    import gen
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[w["dtype"]]
    d, seed = w["d"], w["seed"]
    Q = gen.to_device(gen.tokens(seed, gen.S_QUERY, 0, w["q_len"], d, w["dtype"]), w["dtype"],
                      device)
    if w["kind"] == "fixed":
        B, nd = w["B"], w["nd"]
        D = torch.empty((B, nd, d), dtype=tdt, device=device)
        step = max(1, (1 << 28) // (nd * d * esize(w["dtype"])))
        for b0 in range(0, B, step):
            b1 = min(B, b0 + step)
            D[b0:b1] = gen.to_device(gen.tokens(seed, gen.S_DOCS, b0 * nd, (b1 - b0) * nd, d,
                                                w["dtype"]), w["dtype"], device).view(b1 - b0,
                                                                                     nd, d)
        return dict(Q=Q, D=D, offsets=None, n_tokens=B * nd)
    lens = gen.lengths(seed, w["B"])
    off = gen.csr_offsets(lens)
    T = int(off[-1])
    D = torch.empty((T, d), dtype=tdt, device=device)
    step = (1 << 28) // (d * esize(w["dtype"]))
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        D[t0:t1] = gen.to_device(gen.tokens(seed, gen.S_DOCS, t0, t1 - t0, d, w["dtype"]),
                                 w["dtype"], device)
    return dict(Q=Q, D=D, offsets=torch.from_numpy(off).to(device), n_tokens=T,
                offsets_np=off)


def alg_bytes(w, inp) -> int:
    """Bytes the scoring kernel must move at minimum: every document token once, the query
    once, one fp32 score per document, and the CSR offsets."""
    eb = esize(w["dtype"])
    b = inp["n_tokens"] * w["d"] * eb + w["q_len"] * w["d"] * eb + w["B"] * 4
    if inp["offsets"] is not None:
        b += (w["B"] + 1) * 8
    return b


def run_step(ms, w, inp, out):
    if inp["offsets"] is None:
        ms.maxsim_score_fixed(inp["Q"], inp["D"], out=out)
    else:
        ms.maxsim_score(inp["Q"], inp["D"], inp["offsets"], out=out)


def cpu_baseline(w, budget_s: float):
    """Oracle on the host cores over the first docs of the same workload, sized to ~budget_s."""
    import numpy as np

    import gen
    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    seed, d, dt = w["seed"], w["d"], w["dtype"]
    Qh = gen.tokens(seed, gen.S_QUERY, 0, w["q_len"], d, dt)

    def score(n):
        if w["kind"] == "fixed":
            Dh = gen.tokens(seed, gen.S_DOCS, 0, n * w["nd"], d, dt).reshape(n, w["nd"], d)
            t = time.perf_counter()
            oracle.maxsim_fixed(Qh, Dh, dt, nthreads=threads)
        else:
            off = gen.csr_offsets(gen.lengths(seed, w["B"])[:n])
            Dh = gen.tokens(seed, gen.S_DOCS, 0, int(off[-1]), d, dt)
            t = time.perf_counter()
            oracle.maxsim_csr(Qh, Dh, off, dt, nthreads=threads)
        return time.perf_counter() - t

    n0 = min(w["B"], 256)
    t0 = score(n0)
    n = int(min(w["B"], max(n0, n0 * budget_s / max(t0, 1e-6))))
    t = score(n) if n > n0 else t0
    return {"value": round(n / t, 1), "unit": "docs/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of the {w['B']} documents of the same workload "
                      f"(float64 oracle, {t:.1f} s)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 skips it)")
    ap.add_argument("--no-calib", action="store_true", help="skip the stream-read calibration")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the scoring path runs on a single MI355X and "
              "shards across GPUs by documents with no exchange; run it with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

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
    out = torch.empty(w["B"], dtype=torch.float32, device=dev)
    nbytes = alg_bytes(w, inp)

    # Caches: the MI355X L2 + Infinity Cache hold ~288 MiB. Smaller corpora are flushed
    # between steps and their throughput is taken from the kernel events only.
    footprint = inp["D"].numel() * inp["D"].element_size()
    flush = footprint < (1 << 30)
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev) if flush else None

    for _ in range(args.warmup):
        run_step(ms, w, inp, out)
        if flush:
            scratch.zero_()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        run_step(ms, w, inp, out)
        ends[i].record(stream)
        if flush:
            scratch.zero_()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_ms = sum(kern_ms) / len(kern_ms)
    log(f"timed {args.steps} steps: wall {wall * 1e3 / args.steps:.4f} ms/step, "
        f"kernel avg {avg_ms:.4f} ms, min {min(kern_ms):.4f} ms")

    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    if flush:
        value = w["B"] / (avg_ms * 1e-3)
        ms_per_step = avg_ms
    else:
        value = w["B"] * args.steps / wall
        ms_per_step = wall * 1e3 / args.steps

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE)).get(args.workload)
        if rec and rec.get("kernel_hash") == kernel_hash():
            traffic = rec.get("bytes_per_launch")

    context = {"kernel_ms_avg": round(avg_ms, 5), "kernel_ms_min": round(min(kern_ms), 5),
               "alg_bytes_per_launch": nbytes}
    if not args.no_calib:
        buf = torch.empty(1 << 30, dtype=torch.int32, device=dev)  # 4 GiB
        buf.fill_(1)
        sink = torch.zeros(65536, dtype=torch.int32, device=dev)
        for _ in range(3):
            ms.calib_read(buf, sink)
        cs = [torch.cuda.Event(enable_timing=True) for _ in range(10)]
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(10)]
        for i in range(10):
            cs[i].record(stream)
            ms.calib_read(buf, sink)
            ce[i].record(stream)
        torch.cuda.synchronize()
        cal_ms = sorted(s.elapsed_time(e) for s, e in zip(cs, ce))[5]
        stream_gbs = buf.numel() * 4 / (cal_ms * 1e-3) / 1e9
        context["stream_read_GBps"] = round(stream_gbs, 1)
        context["frac_of_stream_read"] = round(achieved / stream_gbs, 4)
        del buf
        log(f"stream-read ceiling {stream_gbs:.0f} GB/s")

    cpu = None
    if args.cpu_budget > 0:
        log("timing the CPU oracle baseline ...")
        cpu = cpu_baseline(w, args.cpu_budget)
        log(f"cpu baseline {cpu}")

    cfg = {"workload": args.workload, "kind": w["kind"], "n_docs": w["B"], "q_len": w["q_len"],
           "d": w["d"], "storage": w["dtype"]}
    if w["kind"] == "fixed":
        cfg["nd"] = w["nd"]
    else:
        cfg["n_tokens"] = inp["n_tokens"]
        cfg["lengths"] = "lognormal median 70 sigma 0.5 clipped 8..512"
    line = {
        "metric": METRIC if args.workload == DEFAULT else f"docs/s, MaxSim {args.workload}",
        "value": round(value, 1),
        "unit": "docs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded unit-norm Gaussian token embeddings)",
        "config": cfg,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "context": context,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
