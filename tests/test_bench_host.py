"""Host logic of bench.py, no GPU: the timing-event plan, the algorithmic work each roofline
divides by, the bound of each workload, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("steps,kernels,flush", [(1, 1, False), (4, 1, False), (4, 3, False),
                                                 (3, 1, True), (5, 3, True), (50, 1, False)])
def test_boundary_events_recorded_once(steps, kernels, flush):
    """Every event is recorded exactly once, each kernel sits between two consecutive
    records, and without a flush consecutive steps share their boundary event."""
    count, events, closes = bench.boundary_events(steps, kernels, flush)
    recorded = []
    for i in range(steps):
        assert len(events[i]) == kernels + 1
        recorded += events[i][:kernels]
        if closes[i]:
            recorded.append(events[i][-1])
    assert sorted(recorded) == list(range(count))
    for i in range(steps):
        assert events[i] == list(range(events[i][0], events[i][0] + kernels + 1))
        if not flush and i + 1 < steps:
            assert events[i][-1] == events[i + 1][0]
    assert count == steps * kernels + 1 if not flush else count == steps * (kernels + 1)


def _inputs(w):
    """The sizes bench.make_inputs reports, without generating anything."""
    if w["layout"] == "fixed":
        return {"n_tokens": w["B"] * w["nd"], "offsets": None}
    return {"n_tokens": 7_953_858, "offsets": object()}


def test_headline_algorithmic_bytes():
    """Every document byte once, the query once, one fp32 score per document:
    100,000 x 128 x 128 x 2 + 32 x 128 x 2 + 4 x 100,000."""
    w = bench.WORKLOADS["colbert-b100k"]
    work, unit = bench.work_per_launch(w, _inputs(w))
    assert unit == "GB/s"
    assert work == 100_000 * 128 * 128 * 2 + 32 * 128 * 2 + 4 * 100_000 == 3_277_208_192


def test_training_dd_algorithmic_bytes():
    """dD writes one bf16 gradient row per document token and reads the argmax (4 B per query
    token and document), the upstream gradient and the query."""
    w = bench.WORKLOADS["train-colbert-b100k"]
    b = bench.train_dd_bytes(w, _inputs(w))
    assert b == 100_000 * 128 * 128 * 2 + 100_000 * 32 * 4 + 100_000 * 4 + 32 * 128 * 2
    assert b == 3_290_008_192


def test_training_step_roofline_per_launch():
    """A training step's roofline follows the launch that dominates it. The ColPali forward
    with argmax (1024 FLOP per document byte) is matrix-core work on the query-tiled kernel;
    the ColBERT one (32 FLOP per byte) reads the documents and writes the scores and the
    per-token maxima and argmax; dD writes the gradient rows."""
    w = bench.WORKLOADS["train-colpali-b10k"]
    inp = _inputs(w)
    bound, work, unit, fam = bench.train_roofline(w, inp, "maxsim_argmax")
    assert (bound, unit, fam) == ("mfma", "TFLOP/s", "tiled")
    assert work == 2 * 1024 * 10_000 * 1024 * 128
    w = bench.WORKLOADS["train-colbert-b100k"]
    inp = _inputs(w)
    bound, work, unit, fam = bench.train_roofline(w, inp, "maxsim_argmax")
    assert (bound, unit, fam) == ("hbm", "GB/s", "dense")
    assert work == 100_000 * 128 * 128 * 2 + 32 * 128 * 2 + 100_000 * 4 + 100_000 * 32 * 8
    assert bench.train_roofline(w, inp, "backward_dd") == ("hbm", bench.train_dd_bytes(w, inp),
                                                           "GB/s", "train")


def test_matrix_core_work_counts_every_query():
    w = bench.WORKLOADS["batch-colbert-q32-b100k"]
    work, unit = bench.work_per_launch(w, _inputs(w))
    assert unit == "TFLOP/s" and work == 2 * 32 * 32 * 100_000 * 128 * 128
    w = bench.WORKLOADS["colpali-i8-b10k"]
    work, unit = bench.work_per_launch(w, _inputs(w))
    assert unit == "TOP/s" and work == 2 * 1024 * 10_000 * 1024 * 128


def test_several_query_pass_below_the_ridge_counts_bytes():
    """8 ColBERT queries of 32 tokens: 256 FLOP per document byte, below the bf16 ridge
    (2.5 PFLOP/s over 8 TB/s = 312.5), so HBM bounds it; every query and score counts."""
    w = bench.WORKLOADS["batch-colbert-q8-b100k"]
    assert bench.intensity(w) == 256.0
    work, unit = bench.work_per_launch(w, _inputs(w))
    assert unit == "GB/s"
    assert work == 100_000 * 128 * 256 + 8 * (32 * 128 * 2 + 100_000 * 4)
    assert bench.kernel_family(w) == "dbatch"
    assert bench.kernel_family(bench.WORKLOADS["batch-colbert-q32-b100k"]) == "tiled"


def test_int8_short_query_bytes_count_the_scales():
    """INT8 ColBERT shape: one byte per element plus an fp32 scale per document and query
    token, the fp32 score per document."""
    w = bench.WORKLOADS["colbert-i8-b100k"]
    work, unit = bench.work_per_launch(w, _inputs(w))
    assert unit == "GB/s"
    assert work == 100_000 * 128 * (128 + 4) + 32 * (128 + 4) + 100_000 * 4
    assert bench.kernel_family(w) == "dense"


@pytest.mark.parametrize("name,bound", [("colbert-b100k", "hbm"), ("csr-bf16", "hbm"),
                                        ("colbert-i8-b100k", "hbm"),
                                        ("colpali-bf16-b10k", "mfma"), ("colpali-i8-b10k", "mfma"),
                                        ("batch-colbert-q8-b100k", "hbm"),
                                        ("batch-colbert-q32-b100k", "mfma"), ("csr-pq", "lds"),
                                        ("colbert-fp32", "hbm"), ("colpali-i8-b175k", "mfma"),
                                        ("train-csr", "hbm")])
def test_bound_of_each_family(name, bound):
    assert bench.bound_of(bench.WORKLOADS[name]) == bound


def test_peaks_are_the_published_and_derived_ones():
    assert bench.HBM_PEAK_GBS == 8000.0
    assert bench.LDS_PEAK_GBS == pytest.approx(256 * 256 * 2.4)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
