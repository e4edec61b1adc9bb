"""Pins for oracle.e4m3 against facts fixed outside the oracle.

* the OCP E4M3 landmark table (tests/golden/e4m3fn_landmarks.txt);
* torch's CPU float8_e4m3fn decode of all 256 codes (an independent library);
* brute-force nearest-value search with ties to the even code;
* torch's CPU float8 cast (round-to-nearest-even, non-saturating) after a +-448 clamp;
* round trip, saturation, signed zero and monotonicity.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import e4m3


def _landmarks(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "e4m3fn_landmarks.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()[:2]
                rows.append((int(code, 16), float(val)))
    return rows


def test_decode_landmarks(golden_dir):
    rows = _landmarks(golden_dir)
    assert len(rows) >= 14
    for code, val in rows:
        got = e4m3.decode(np.array([code], np.uint8))[0]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3.decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_ours, nan_ref)
    assert set(np.flatnonzero(nan_ours)) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref])
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(ref[~nan_ref]))


def test_format_constants():
    vals = e4m3.finite_values()
    assert len(vals) == 127
    assert vals.max() == 448.0 and vals[0x7E] == 448.0
    assert vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6
    assert np.all(np.diff(vals) > 0)  # codes 0x00..0x7E are increasing


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3.decode(codes).astype(np.float32)
    back = e4m3.encode(vals)
    assert np.array_equal(back, codes)


def _brute_force_encode(v):
    """Nearest of the 127 non-negative values by exhaustive distance, ties -> even code."""
    table = [math.ldexp(m, -9) for m in range(8)]
    table += [(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)][:119]
    assert len(table) == 127 and table[-1] == 448.0
    out = []
    for x in v:
        a = min(abs(float(x)), 448.0)
        best, best_d = None, None
        for code, t in enumerate(table):
            d = abs(a - t)
            if best is None or d < best_d or (d == best_d and code % 2 == 0):
                best, best_d = code, d
        out.append(best | (0x80 if math.copysign(1.0, float(x)) < 0 else 0))
    return np.array(out, dtype=np.uint8)


def _decision_points():
    vals = e4m3.finite_values()
    mids = (vals[:-1] + vals[1:]) / 2  # every rounding boundary, exact in float32
    pts = [vals, mids, [464.0, 448.0 + 2 ** -15, 500.0, 1e30, 2.0 ** -11, 2.0 ** -12, 0.0]]
    pts = np.concatenate([np.asarray(p, np.float64) for p in pts]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    down = np.nextafter(pts, np.float32(0))
    allp = np.concatenate([pts, up, down])
    return np.concatenate([allp, -allp]).astype(np.float32)


def test_encode_matches_brute_force_at_every_boundary():
    v = _decision_points()
    assert np.array_equal(e4m3.encode(v), _brute_force_encode(v))


def test_encode_matches_brute_force_random():
    rng = np.random.default_rng(7)
    v = (rng.uniform(-1, 1, 4000) * np.exp2(rng.uniform(-14, 10, 4000))).astype(np.float32)
    assert np.array_equal(e4m3.encode(v), _brute_force_encode(v))


def _torch_encode(v):
    t = torch.from_numpy(np.asarray(v, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(11)
    n = 1 << 20
    mag = np.exp2(rng.uniform(-24, 12, n))
    v = (np.where(rng.random(n) < 0.5, -1, 1) * mag).astype(np.float32)
    v = np.concatenate([v, _decision_points()])
    assert np.array_equal(e4m3.encode(v), _torch_encode(v))


def test_encode_dense_bf16_grid_matches_torch():
    # every finite bf16 value (as float32), a 16-bit exhaustive sweep of the encode
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(e4m3.encode(f), _torch_encode(f))


def test_saturation_and_ties():
    cases = [
        (448.0, 0x7E), (449.0, 0x7E), (464.0, 0x7E), (465.0, 0x7E), (1e30, 0x7E), (-1e30, 0xFE),
        (1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
        (-(2.0 ** -12), 0x80), (-0.0, 0x80), (0.0, 0x00), (7.5 * 2.0 ** -9, 0x08),
    ]
    for x, code in cases:
        assert e4m3.encode(np.array([x], np.float32))[0] == code, x


def test_encode_monotone_and_odd():
    v = np.sort(np.exp2(np.linspace(-16, 9.5, 200001)).astype(np.float32))
    dec = e4m3.decode(e4m3.encode(v))
    assert np.all(np.diff(dec) >= 0)
    assert np.array_equal(e4m3.encode(-v), e4m3.encode(v) ^ 0x80)


def test_encode_rejects_non_finite():
    for bad in (np.inf, -np.inf, np.nan):
        with pytest.raises(ValueError):
            e4m3.encode(np.array([1.0, bad], np.float32))
