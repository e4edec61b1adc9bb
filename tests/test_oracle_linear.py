"""Pins for oracle.linear (exact FP8 product and the scale/bias epilogue).

* the float64 product equals an int64 dot of the codes' integer values (units of 2^-9);
* a pure-Python triple loop on small non-square shapes (catches transposed operands);
* A = 0 gives exactly the bias; one-hot unit weights select single columns;
* the quantised linear stays close to the unquantised bf16 linear (information level).
"""

import numpy as np
import torch

from oracle import e4m3, linear, quant
from workloads import bf16_bits, make_case


def _int_values(codes):
    """dec(code) * 2^9 as int64, computed from the bits by integer arithmetic only."""
    c = codes.astype(np.int64)
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0))
    return np.where(s == 1, -mag, mag)


def _random_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    c[(c & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    return c.astype(np.uint8)


def test_int_values_helper_matches_decode():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(_int_values(codes).astype(np.float64), e4m3.decode(codes) * 512.0)


def test_gemm_exact_equals_int64_dot():
    rng = np.random.default_rng(1)
    for m, n, k in [(3, 5, 16), (17, 9, 272), (8, 33, 2048), (4, 4, 8192)]:
        qa, qw = _random_codes(rng, (m, k)), _random_codes(rng, (n, k))
        acc = linear.gemm_exact(qa, qw)
        exact = _int_values(qa) @ _int_values(qw).T  # units of 2^-18, no rounding
        assert np.array_equal(acc * 2.0 ** 18, exact.astype(np.float64))
        assert np.all(np.abs(exact) < 2 ** 53)


def test_worst_case_magnitudes_exact():
    k = 8192
    qa = np.full((2, k), 0x7E, np.uint8)
    qw = np.full((3, k), 0x7E, np.uint8)
    qw[1] = 0xFE
    acc = linear.gemm_exact(qa, qw)
    assert np.all(acc[:, 0] == 448.0 * 448.0 * k) and np.all(acc[:, 1] == -448.0 * 448.0 * k)


def test_linear_matches_python_loops():
    case = make_case(5, 7, 48, seed=4, kind="outlier", outliers=2)
    wq, ws = quant.quant_rows(bf16_bits(case.w))
    out, qa, sa = linear.linear_ref(bf16_bits(case.a), wq, ws, bf16_bits(case.bias))
    da, dw = e4m3.decode(qa), e4m3.decode(wq)
    b = case.bias.double().numpy()
    for i in range(5):
        for j in range(7):
            acc = 0.0
            for kk in range(48):
                acc += da[i, kk] * dw[j, kk]
            ref = acc * float(sa[i]) * float(ws[j]) + b[j]
            assert out[i, j] == ref or abs(out[i, j] - ref) <= 1e-12 * (abs(ref) + 1)


def test_zero_activation_gives_bias():
    case = make_case(4, 32, 64, seed=2)
    wq, ws = quant.quant_rows(bf16_bits(case.w))
    zero = np.zeros((4, 64), np.uint16)
    out, qa, sa = linear.linear_ref(zero, wq, ws, bf16_bits(case.bias))
    assert np.all(sa == 0) and np.all(qa == 0)
    assert np.array_equal(out, np.broadcast_to(case.bias.double().numpy(), out.shape))


def test_one_hot_weights_select_columns():
    m, k = 6, 64
    case = make_case(m, 16, k, seed=8, with_bias=False)
    qa, sa = quant.quant_rows(bf16_bits(case.a))
    qw = np.zeros((16, k), np.uint8)
    cols = np.arange(16) * 3
    qw[np.arange(16), cols] = 0x38  # 1.0
    sw = np.full(16, 0.5, np.float32)
    out = linear.linear_ref_fp8(qa, sa, qw, sw)
    expect = e4m3.decode(qa)[:, cols] * sa[:, None].astype(np.float64) * 0.5
    assert np.array_equal(out, expect)


def test_bias_none_and_scales_broadcast_along_the_right_axes():
    rng = np.random.default_rng(3)
    qa, qw = _random_codes(rng, (3, 32)), _random_codes(rng, (5, 32))
    sa = np.array([1, 2, 4], np.float32)
    sw = np.array([1, 10, 100, 1000, 10000], np.float32)
    acc = linear.gemm_exact(qa, qw)
    out = linear.linear_ref_fp8(qa, sa, qw, sw)
    for i in range(3):
        for j in range(5):
            assert out[i, j] == acc[i, j] * sa[i] * sw[j]


def test_close_to_unquantised_linear():
    case = make_case(64, 128, 256, seed=0, kind="outlier", outliers=2)
    wq, ws = quant.quant_rows(bf16_bits(case.w))
    out, _, _ = linear.linear_ref(bf16_bits(case.a), wq, ws, bf16_bits(case.bias))
    ref = torch.nn.functional.linear(case.a.double(), case.w.double(), case.bias.double()).numpy()
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 0.08, rel
