"""Pins for oracle.w8a16 (the FP8 weight-only linear).

* brute force with exact rational arithmetic on small non-square shapes;
* where the per-token quantiser is the identity (rows of e4m3fn values whose largest
  magnitude is 448, so s = 1), the weight-only result equals the W8A8 oracle's, whose
  product is pinned to an int64 dot of the codes;
* a = 0 gives exactly the bias; one-hot rows of a select one dequantised weight column;
* the result scales with the weight scale, per output channel.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import e4m3, linear, quant, w8a16
from workloads import bf16_bits, make_case


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c.astype(np.uint8)


def _bits(x):
    return bf16_bits(torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16))


def brute_force(a_bits, qw, sw, bias_bits):
    a = quant.bf16_bits_to_f32(a_bits)
    w = e4m3.decode(qw)
    b = quant.bf16_bits_to_f32(bias_bits) if bias_bits is not None else None
    m, k = a.shape
    n = w.shape[0]
    out = np.empty((m, n))
    for i in range(m):
        for j in range(n):
            s = sum(Fraction(float(a[i, t])) * Fraction(float(w[j, t])) for t in range(k))
            s = s * Fraction(float(np.float32(sw[j])))
            if b is not None:
                s += Fraction(float(b[j]))
            out[i, j] = float(s)
    return out


def test_matches_exact_rational_brute_force():
    rng = np.random.default_rng(3)
    for m, n, k in [(3, 5, 16), (4, 7, 48), (2, 3, 160)]:
        a = _bits(rng.standard_normal((m, k)) * np.exp2(rng.integers(-20, 20, (m, 1))))
        qw = _codes(rng, (n, k))
        sw = (rng.random(n) * 0.01).astype(np.float32)
        b = _bits(rng.standard_normal(n) * 0.1)
        got = w8a16.w8a16_ref(a, qw, sw, b)
        exp = brute_force(a, qw, sw, b)
        assert np.allclose(got, exp, rtol=1e-13, atol=1e-30)


def test_equals_w8a8_where_the_activation_quant_is_the_identity():
    rng = np.random.default_rng(4)
    m, n, k = 24, 40, 272
    qa = _codes(rng, (m, k))
    qa[:, 5] = 0x7E  # every row reaches 448, so s = 448 / 448 = 1 and x / s = x
    a_bits = _bits(e4m3.decode(qa))  # e4m3 values are exact in bf16
    q_chk, s_chk = quant.quant_rows(a_bits)
    assert np.all(s_chk == 1.0) and np.array_equal(q_chk, qa)
    qw = _codes(rng, (n, k))
    sw = (rng.random(n) * 0.02).astype(np.float32)
    b = _bits(rng.standard_normal(n))
    ref8, _, _ = linear.linear_ref(a_bits, qw, sw, b)
    assert np.array_equal(w8a16.w8a16_ref(a_bits, qw, sw, b), ref8)


def test_zero_activation_and_one_hot_rows():
    rng = np.random.default_rng(5)
    n, k = 12, 64
    qw = _codes(rng, (n, k))
    sw = (rng.random(n) + 0.5).astype(np.float32)
    b = _bits(rng.standard_normal(n))
    zero = np.zeros((3, k), np.uint16)
    assert np.array_equal(w8a16.w8a16_ref(zero, qw, sw, b), np.tile(quant.bf16_bits_to_f32(b), (3, 1)))
    one_hot = np.zeros((k, k), np.float32)
    np.fill_diagonal(one_hot, 1.0)
    out = w8a16.w8a16_ref(_bits(one_hot), qw, sw)  # row t selects column t of the dequantised weight
    assert np.array_equal(out, (e4m3.decode(qw) * sw.astype(np.float64)[:, None]).T)


def test_scales_act_per_output_channel():
    case = make_case(8, 16, 64, seed=2, kind="normal")
    qw, sw = quant.quant_weights_per_channel(bf16_bits(case.w))
    a = bf16_bits(case.a)
    base = w8a16.w8a16_ref(a, qw, sw)
    sw2 = sw.copy()
    sw2[3] *= np.float32(4.0)
    out = w8a16.w8a16_ref(a, qw, sw2)
    assert np.array_equal(out[:, 3], 4.0 * base[:, 3])
    assert np.array_equal(np.delete(out, 3, axis=1), np.delete(base, 3, axis=1))


def test_close_to_the_unquantised_linear():
    # information level: weight-only quantisation keeps the product within a few percent
    case = make_case(16, 64, 512, seed=6, kind="normal")
    qw, sw = quant.quant_weights_per_channel(bf16_bits(case.w))
    got = w8a16.w8a16_ref(bf16_bits(case.a), qw, sw)
    full = case.a.double().numpy() @ case.w.double().numpy().T
    assert np.linalg.norm(got - full) / np.linalg.norm(full) < 0.05
