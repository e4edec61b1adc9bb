"""Pins for oracle.quant (per-token and per-channel row quantisation).

* hand-worked rows with exact power-of-two scales (tests/golden/quant_rows_worked.txt);
* an independent torch CPU implementation: fp32 amax / 448, fp32 division, clamp,
  torch's float8_e4m3fn cast;
* invariants: the amax element codes to +-448, odd symmetry, monotonicity within a
  row, exact power-of-two rescaling, the error bound of a 3-bit mantissa, zero rows;
* bf16 -> float32 against torch's own conversion.
"""

import os

import numpy as np
import pytest
import torch

from oracle import e4m3, quant
from workloads import bf16_bits, make_case, make_config


def _worked_rows(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "quant_rows_worked.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            s, xs, codes = [p.strip() for p in line.split("|")]
            rows.append((float.fromhex(s), [float.fromhex(x) for x in xs.split()],
                         [int(c, 16) for c in codes.split()]))
    return rows


def _bits_of(values):
    t = torch.tensor(values, dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(t.float(), torch.tensor(values, dtype=torch.float32)), "not exact in bf16"
    return bf16_bits(t)


def test_worked_rows(golden_dir):
    rows = _worked_rows(golden_dir)
    assert len(rows) == 4
    for s, xs, codes in rows:
        q, sc = quant.quant_rows(_bits_of([xs]))
        assert sc[0] == np.float32(s)
        assert list(q[0]) == codes, (xs, list(map(hex, q[0])))


def _torch_quant(x_bf16):
    x = x_bf16.float()
    s = x.abs().amax(dim=1) / torch.tensor(448.0, dtype=torch.float32)
    q = torch.empty(x.shape, dtype=torch.uint8)
    nz = s > 0
    q[nz] = (x[nz] / s[nz, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    q[~nz] = torch.where(torch.signbit(x[~nz]), 0x80, 0).to(torch.uint8)
    return q.numpy(), s.numpy()


@pytest.mark.parametrize("m,k,kind", [(64, 256, "outlier"), (37, 2048, "gelu"), (5, 8192, "outlier"),
                                      (129, 48, "normal")])
def test_matches_torch_quant(m, k, kind):
    case = make_case(m, 16, k, seed=3, kind=kind)
    q, s = quant.quant_rows(bf16_bits(case.a))
    tq, ts = _torch_quant(case.a)
    assert np.array_equal(s, ts)
    assert np.array_equal(q, tq)


def test_tiny_config_matches_torch():
    cfg = make_config("tiny")
    for t in (cfg["activations"]["a"], cfg["weights"]["linear"]):
        q, s = quant.quant_rows(bf16_bits(t))
        tq, ts = _torch_quant(t)
        assert np.array_equal(q, tq) and np.array_equal(s, ts)


def test_extreme_magnitude_rows_match_torch():
    rng = np.random.default_rng(5)
    rows = []
    for e in (-133, -126, -100, -80, -40, 0, 40, 100, 120):
        r = rng.standard_normal(300).astype(np.float32) * np.float32(2.0 ** e)
        rows.append(r)
    x = torch.from_numpy(np.stack(rows)).to(torch.bfloat16)
    q, s = quant.quant_rows(bf16_bits(x))
    tq, ts = _torch_quant(x)
    assert np.array_equal(s, ts) and np.array_equal(q, tq)


def hard_quotient_rows(count=200, seed=0):
    """Rows [amax, x...] whose quotients x / s and x * (1 / s) round to different codes.

    Found with plain numpy arithmetic and torch's float8 cast (no oracle code): these are
    the elements where a divide-free shortcut would go wrong, so the oracle is held to
    the correctly rounded quotient exactly where it matters.
    """
    pat = np.arange(1 << 16, dtype=np.uint32)
    x = (pat << 16).view(np.float32)
    x = x[np.isfinite(x)]

    def enc(v):
        return torch.from_numpy(np.clip(v, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn) \
            .view(torch.uint8).numpy()

    rows = []
    rng = np.random.default_rng(seed)
    for a_bits in rng.integers(0x3000, 0x5000, count):
        amax = np.float32((np.uint32(a_bits) << 16).view(np.float32))
        xs = x[np.abs(x) <= amax]
        s = np.float32(amax / np.float32(448))
        r = np.float32(np.float32(1) / s)
        d = np.flatnonzero(enc((xs / s).astype(np.float32)) != enc((xs * r).astype(np.float32)))
        if len(d):
            row = np.zeros(8, np.float32)
            row[0] = amax
            picks = xs[d[:7]]
            row[1:1 + len(picks)] = picks
            rows.append(row)
    return np.stack(rows)


def test_hard_quotients_match_torch():
    rows = hard_quotient_rows()
    assert len(rows) >= 10
    x = torch.from_numpy(rows).to(torch.bfloat16)
    q, s = quant.quant_rows(bf16_bits(x))
    tq, ts = _torch_quant(x)
    assert np.array_equal(s, ts) and np.array_equal(q, tq)


def test_invariants():
    case = make_case(96, 16, 1024, seed=9, kind="outlier")
    bits = bf16_bits(case.a)
    x = quant.bf16_bits_to_f32(bits)
    q, s = quant.quant_rows(bits)
    # the amax element of every row codes to +-448
    idx = np.argmax(np.abs(x), axis=1)
    assert np.all((q[np.arange(len(idx)), idx] & 0x7F) == 0x7E)
    # odd symmetry
    qn, sn = quant.quant_rows(bits ^ np.uint16(0x8000))
    assert np.array_equal(sn, s) and np.array_equal(qn, q ^ 0x80)
    # monotone within each row
    dec = e4m3.decode(q)
    for r in range(x.shape[0]):
        order = np.argsort(x[r], kind="stable")
        assert np.all(np.diff(dec[r][order]) >= 0)
    # exact rescaling by a power of two (no under- or overflow here)
    for j in (-20, -3, 5, 30):
        qj, sj = quant.quant_rows_f32(x * np.float32(2.0 ** j))
        assert np.array_equal(qj, q) and np.array_equal(sj, s * np.float32(2.0 ** j))
    # a 3-bit mantissa bounds the relative error by 2^-4 in the normal range
    recon = dec * s[:, None]
    normal = np.abs(x) / s[:, None] >= 2.0 ** -6
    assert np.all(np.abs(x - recon)[normal] <= 2.0 ** -4 * np.abs(x)[normal] * (1 + 1e-6))
    sub = ~normal
    assert np.all(np.abs(x - recon)[sub] <= 2.0 ** -10 * np.broadcast_to(s[:, None], x.shape)[sub] * (1 + 1e-6))


def test_zero_rows_and_signed_zero():
    x = np.zeros((3, 8), np.float32)
    x[1, 2] = -0.0
    x[2] = [0, -0.0, 1.0, -1.0, 0, 0, 0, 0]
    q, s = quant.quant_rows_f32(x)
    assert s[0] == 0 and s[1] == 0 and s[2] == np.float32(1.0 / 448.0)
    assert q[1, 2] == 0x80 and np.all(np.delete(q[1], 2) == 0)
    assert list(q[2, :4]) == [0x00, 0x80, 0x7E, 0xFE]


def test_bf16_bits_to_f32_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = quant.bf16_bits_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert np.all(same)


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        quant.quant_rows_f32(np.array([[1.0, np.inf]], np.float32))
