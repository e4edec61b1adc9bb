"""Host-side summaries of rocprofv3 output (fp8_w8a8_quantized_token_amd.profiling)."""
import csv
import json

import pytest

from fp8_w8a8_quantized_token_amd import profiling

TRACE_FIELDS = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]


def _write_trace(path, launches):
    """launches: (name, start_ns, end_ns); written in shuffled order (the reader sorts)."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_FIELDS)
        w.writeheader()
        for name, s, e in reversed(launches):
            w.writerow({"Kind": "KERNEL_DISPATCH", "Kernel_Name": name, "Start_Timestamp": s, "End_Timestamp": e})


def test_runs_back_to_back_and_after(tmp_path):
    t = 0
    launches = []

    def add(name, dur, gap):
        nonlocal t
        t += gap
        launches.append((name, t, t + dur))
        t += dur

    for _ in range(5):  # steps: Q then G
        add("quant<2>", 9_000, 500)
        add("gemm<false>", 68_000, 600)
    for _ in range(4):  # G back to back
        add("gemm<false>", 70_000, 200)
    add("other", 1_000, 100)
    for _ in range(3):  # Q back to back
        add("quant<2>", 7_000, 800)
    p = tmp_path / "trace.csv"
    _write_trace(p, launches)

    b2b = profiling.runs(str(p), "gemm<false>", min_run=2)
    # the first back-to-back GEMM follows a step's GEMM, so the stretch is 4 launches
    assert [r["launches"] for r in b2b] == [4]
    assert b2b[0]["mean_us"] == pytest.approx(70.0) and b2b[0]["mean_gap_before_us"] == pytest.approx(0.2)

    step = profiling.runs(str(p), "gemm<false>", after="quant<2>", min_run=2)
    assert [r["launches"] for r in step] == [5]
    assert step[0]["mean_us"] == pytest.approx(68.0) and step[0]["mean_gap_before_us"] == pytest.approx(0.6)

    q = profiling.runs(str(p), "quant<2>", min_run=2)
    assert [r["launches"] for r in q] == [2]  # the first of the three follows "other"
    assert q[0]["median_us"] == pytest.approx(7.0)
    assert profiling.runs(str(p), "quant<2>", min_run=3) == []

    text = profiling.runs_markdown(step, "gemm<false>", "quant<2>", "cmd")
    assert "| 5 | 68.00 | 68.00 | 0.60 |" in text


def test_stats_markdown(tmp_path):
    p = tmp_path / "stats.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": "void fp8w8a8::(anonymous namespace)::gemm_fp8_kernel<1>(GemmArgs)", "Calls": 3,
                    "AverageNs": 70500.0, "MinNs": 70000, "MaxNs": 71000, "Percentage": 90.0})
    text = profiling.stats_markdown(str(p), "rocprofv3 ...")
    assert "| `void gemm_fp8_kernel<1>(GemmArgs)` | 3 | 70.50 | 70.00 | 71.00 | 90.0 |" in text


def test_committed_traffic_record_is_well_formed():
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    t = json.load(open(os.path.join(root, "profiles", "gemm_fp8_ffn_up_traffic.json")))
    assert t["hbm_bytes_per_launch"] == pytest.approx(t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"])
    assert t["launches"] > 0 and len(t["source_sha256"]) == 64
