"""Pins for oracle.e5m2 against facts fixed outside the oracle.

* the OCP E5M2 landmark table (tests/golden/e5m2_landmarks.txt);
* torch's CPU float8_e5m2 decode of all 256 codes (an independent library);
* brute-force nearest-value search with ties to the even code at every boundary;
* torch's CPU float32 -> float8_e5m2 cast (round to nearest even) after a +-57344 clamp,
  on log-uniform values and on every finite bf16 value;
* saturation, subnormal ties and signed zero.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import e5m2


def _landmarks(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "e5m2_landmarks.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()[:2]
                rows.append((int(code, 16), float(val)))
    return rows


def test_decode_landmarks(golden_dir):
    rows = _landmarks(golden_dir)
    assert len(rows) >= 15
    for code, val in rows:
        got = e5m2.decode(np.array([code], np.uint8))[0]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e5m2.decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], ref[fin]) and np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_format_constants():
    vals = e5m2.finite_values()
    assert len(vals) == 124 and vals[-1] == 57344.0
    assert vals[1] == 2.0 ** -16 and vals[4] == 2.0 ** -14
    assert np.all(np.diff(vals) > 0)


def _brute(v):
    vals = e5m2.finite_values()
    a = min(abs(float(v)), 57344.0)
    d = np.abs(vals - a)
    best = np.flatnonzero(d == d.min())
    code = int(best[0]) if len(best) == 1 else int(best[0] if best[0] % 2 == 0 else best[1])
    return code | (0x80 if math.copysign(1.0, float(v)) < 0 else 0)


def test_encode_matches_brute_force_at_every_boundary():
    vals = e5m2.finite_values()
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0))])
    pts = np.concatenate([pts, -pts, np.float32([60000.0, 1e30, 2.0 ** -18, -0.0])])
    got = e5m2.encode(pts)
    exp = np.array([_brute(v) for v in pts], np.uint8)
    assert np.array_equal(got, exp)


def _torch_cast(v):
    t = torch.from_numpy(np.clip(np.asarray(v, np.float32), -57344.0, 57344.0))
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_encode_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(0)
    v = (np.exp2(rng.uniform(-20, 17, 1_000_000)) * rng.choice([-1, 1], 1_000_000)).astype(np.float32)
    assert np.array_equal(e5m2.encode(v), _torch_cast(v))
    bits = np.arange(1 << 16, dtype=np.uint32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]
    allbf = (bits << 16).view(np.float32)
    assert np.array_equal(e5m2.encode(allbf), _torch_cast(allbf))


def test_saturation_ties_and_zero():
    enc = lambda x: int(e5m2.encode(np.float32([x]))[0])  # noqa: E731
    assert enc(57344.0) == 0x7B and enc(1e9) == 0x7B and enc(-1e9) == 0xFB
    assert enc(61440.0) == 0x7B  # the would-be next value (the infinity position) saturates
    assert enc(2.0 ** -17) == 0x00 and enc(3 * 2.0 ** -17) == 0x02  # subnormal ties to even
    assert enc(1.125) == 0x3C and enc(1.375) == 0x3E  # 1 + 1/8 -> 1.0 (even); 1 + 3/8 -> 1.5 (even)
    assert enc(-0.0) == 0x80 and enc(-2.0 ** -20) == 0x80
    with pytest.raises(ValueError):
        e5m2.encode(np.float32([np.inf]))
