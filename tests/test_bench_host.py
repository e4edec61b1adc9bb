"""Host-side logic of bench.py: the amd-smi clock parser, percentiles, the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _clk(v):
    return {"clk": {"value": v, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
            "max_clk": {"value": 2400, "unit": "MHz"}, "clk_locked": "DISABLED", "deep_sleep": "ENABLED"}


def test_smi_clock_parser_means_over_xcds():
    clock = {f"gfx_{i}": _clk(1900 + 10 * i) for i in range(8)}
    clock["mem_0"] = _clk(2000)
    clock["vclk_0"] = _clk(29)
    text = json.dumps({"gpu_data": [{"gpu": 0, "clock": clock}]})
    assert bench._smi_clocks(text) == (1935.0, 2000.0)


def test_smi_clock_parser_list_form_and_missing_mem():
    text = json.dumps([{"gpu": 0, "clock": {"gfx_0": _clk(2100), "gfx_1": _clk(2000)}}])
    assert bench._smi_clocks(text) == (2050.0, None)


def test_percentile_nearest_rank():
    xs = sorted([5.0, 1.0, 4.0, 2.0, 3.0])
    assert bench.pct(xs, 0) == 1.0 and bench.pct(xs, 50) == 3.0 and bench.pct(xs, 100) == 5.0
    assert bench.pct(xs, 10) == 1.0 and bench.pct(xs, 90) == 5.0
    assert bench.pct([7.0], 90) == 7.0


def test_fp8_peak_per_clock_matches_published_peak():
    # 256 CUs x 8192 flop per clock at 2.4 GHz is the published 5.0 PFLOP/s dense FP8.
    assert bench.N_CUS * bench.FP8_FLOP_PER_CU_CLK * 2.4e9 / 1e12 == pytest.approx(bench.PEAK_FP8_TFLOPS, rel=0.01)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
