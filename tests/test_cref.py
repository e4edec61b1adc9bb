"""Pins for the C statement of the quantiser (oracle/csrc/quant_ref.c) against oracle.quant.

The C oracle exists for sweeps too large for numpy (the exhaustive bf16 pair sweep in
test_gpu_quant.py); here it must agree bit for bit with the pinned Python oracle.
"""

import numpy as np
import torch

from oracle import cref, e4m3, quant
from workloads import bf16_bits, make_case


def test_encode_matches_python_on_decision_points():
    vals = e4m3.finite_values()
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, [464.0, 500.0, 1e30, 2.0 ** -11, 0.0]]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0))])
    pts = np.concatenate([pts, -pts, np.array([-0.0], np.float32)])
    c = np.array([cref.lib().oracle_encode_e4m3fn(float(v)) for v in pts], np.uint8)
    assert np.array_equal(c, e4m3.encode(pts))


def test_rows_match_python_random_and_extreme():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 300)).astype(np.float32)
    x *= np.exp2(rng.integers(-133, 120, (64, 1))).astype(np.float32)
    x[3] = 0.0
    x[4, ::2] = -0.0
    bits = bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
    q1, s1 = cref.quant_rows(bits)
    q2, s2 = quant.quant_rows(bits)
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_rows_match_python_configs():
    for kind, k in (("outlier", 2048), ("gelu", 8192)):
        bits = bf16_bits(make_case(48, 16, k, seed=5, kind=kind).a)
        q1, s1 = cref.quant_rows(bits)
        q2, s2 = quant.quant_rows(bits)
        assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_every_bf16_value_against_sampled_amax():
    # a slice of the exhaustive sweep: every finite bf16 x under 64 amax values
    pat = np.arange(1 << 16, dtype=np.int64)
    mag, sign = pat & 0x7FFF, pat & 0x8000
    rng = np.random.default_rng(3)
    amaxes = np.concatenate([[1, 0x0080, 0x3F80, 0x7F7F], rng.integers(1, 0x7F80, 60)])
    rows = []
    for a in amaxes:
        m = np.where(mag > a, a, mag)
        m = np.where(mag <= 0x7F7F, m, 0)
        rows.append((sign | m).astype(np.uint16))
    bits = np.stack(rows)
    q1, s1 = cref.quant_rows(bits)
    q2, s2 = quant.quant_rows(bits)
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
