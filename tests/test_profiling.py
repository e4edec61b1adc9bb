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


def _write_counters(path, counter, launches):
    """launches: (kernel name, grid size, value KiB)."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, grid, v in launches:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_groups_launches_by_grid_size(tmp_path):
    # one kernel at two shapes (as the quantiser runs on activations and weights): each shape
    # gets its own median, scaled by the 1 GiB copy's reading, with its algorithmic ratio
    cal = [("__amd_rocclr_copyBuffer", 1 << 20, 524288.0)] * 3
    fetch = cal + [("quant_rows_regs<2>", 262144, 16384.0)] * 5 + [("quant_rows_regs<2>", 524288, 32768.0)] * 4
    write = [(n, g, 2 * v if "copy" in n else v / 2) for n, g, v in fetch]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counters(fp, "FETCH_SIZE", fetch)
    _write_counters(wp, "WRITE_SIZE", write)
    t = profiling.traffic(str(fp), str(wp), "quant_rows", groups={524288: (50e6, "weights")})
    assert [g["grid_size"] for g in t["groups"]] == [524288, 262144]
    w, a = t["groups"]
    assert w["launches"] == 4 and a["launches"] == 5
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert w["fetch_bytes_per_launch"] == pytest.approx(32768 * 1024 * 2)
    assert w["write_bytes_per_launch"] == pytest.approx(16384 * 1024)
    assert w["traffic_over_algorithmic"] == pytest.approx((64 + 16) * 1024 * 1024 / 50e6)
    assert t["hbm_bytes_per_launch"] == w["hbm_bytes_per_launch"]
    text = profiling.traffic_markdown(t, "cmd")
    assert "| weights | 524288 | 4 |" in text and "| - | 262144 | 5 |" in text


def test_counters_mfma_busy_share(tmp_path):
    # 3 launches of one shape: GUI-active summed over 8 XCDs, MFMA busy summed over 1024 SIMDs
    p = tmp_path / "c.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for d in range(3):
            row = {"Dispatch_Id": d, "Kernel_Name": "gemm<false>", "Grid_Size": 262144,
                   "Start_Timestamp": 1000, "End_Timestamp": 1000 + 50_000}
            w.writerow(dict(row, Counter_Name="GRBM_GUI_ACTIVE", Counter_Value=8 * 100_000))
            w.writerow(dict(row, Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES", Counter_Value=1024 * 60_000))
            w.writerow(dict(row, Counter_Name="SQ_INSTS_VALU_MFMA_MOPS_F8", Counter_Value=1_000_000))
    recs = profiling.counters(str(p), "gemm", {262144: (5.12e8, "FFN-up")})
    assert len(recs) == 1
    r = recs[0]
    assert r["launches"] == 3 and r["label"] == "FFN-up"
    assert r["mfma_busy"] == pytest.approx(0.6)
    assert r["mfma_flop"] == pytest.approx(5.12e8)
    assert r["duration_us"] == pytest.approx(50.0) and r["gui_clock_ghz"] == pytest.approx(2.0)
    assert "| matrix-core busy share" in profiling.counters_markdown(recs, "cmd")


def test_counters_two_kernels_on_one_grid_size(tmp_path):
    # the persistent 256 x 256 GEMM (256 workgroups) and the 128 x 256 tiles at FFN-down
    # (256 tiles) both launch 131072 work-items: records per kernel, labels by name
    p = tmp_path / "c.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d, (name, busy) in enumerate([("gemm<256, 256, true>", 50_000), ("gemm<128, 256, false>", 70_000)] * 2):
            row = {"Dispatch_Id": d, "Kernel_Name": name, "Grid_Size": 131072}
            w.writerow(dict(row, Counter_Name="GRBM_GUI_ACTIVE", Counter_Value=8 * 100_000))
            w.writerow(dict(row, Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES", Counter_Value=1024 * busy))
    groups = {("<256, 256", 131072): (1.0, "FFN-up"), ("<128, 256", 131072): (2.0, "FFN-down")}
    recs = profiling.counters(str(p), "gemm", groups)
    assert [r["label"] for r in recs] == ["FFN-up", "FFN-down"]
    assert [r["launches"] for r in recs] == [2, 2]
    assert recs[0]["mfma_busy"] == pytest.approx(0.5) and recs[1]["mfma_busy"] == pytest.approx(0.7)
    assert recs[1]["algorithmic_flop"] == 2.0


def test_bench_reports_traffic_only_for_the_current_gemm_sources(tmp_path):
    # the bench's roofline.traffic comes from a committed counter record, and only while
    # the GEMM sources are byte for byte the ones the counters were taken on
    import hashlib
    import bench

    h = hashlib.sha256()
    for p in bench.GEMM_SOURCES:
        h.update(open(p, "rb").read())
    rec = {"hbm_bytes_per_launch": 123456789.0, "gemm_source_sha256": h.hexdigest()}
    good = tmp_path / "good.json"
    good.write_text(json.dumps(rec))
    assert bench.traffic_from_profile(str(good)) == 123456789.0
    stale = tmp_path / "stale.json"
    stale.write_text(json.dumps(dict(rec, gemm_source_sha256="0" * 64)))
    assert bench.traffic_from_profile(str(stale)) is None
    assert bench.traffic_from_profile(str(tmp_path / "missing.json")) is None
