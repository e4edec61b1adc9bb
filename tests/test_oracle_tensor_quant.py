"""Pins for oracle.tensor_quant (per-tensor FP8 quantisation, either format, and fp32 dequantisation).

* a one-row tensor quantises exactly like the (separately pinned) per-token quantiser, in e4m3fn;
* a hand-worked tensor with an exact power-of-two scale, in both formats;
* invariants: the amax element maps to the largest finite code, odd symmetry, exact 2^j rescaling,
  the relative error bound of each format on normal-range values, zero tensors;
* dequantisation is the correctly rounded fp32 product: the float64 product of a code's value
  (at most 4 significant bits) and the fp32 scale is exact, and rounding it to fp32 once must agree.
"""

import numpy as np
import pytest
import torch

from oracle import e4m3, e5m2, quant, tensor_quant as tq
from workloads import bf16_bits


def _bits(x):
    return bf16_bits(torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16))


def test_one_row_equals_per_token_quant():
    rng = np.random.default_rng(1)
    for k in (16, 300, 2048):
        x = _bits(rng.standard_normal((1, k)) * np.exp2(rng.integers(-30, 30)))
        q1, s1 = tq.quant_tensor(x, "e4m3fn")
        q2, s2 = quant.quant_rows(x)
        assert np.array_equal(q1, q2) and s1 == s2[0]


def test_worked_tensor_power_of_two_scale():
    # amax = 448 * 2^-3 = 56 -> s = 2^-3 exactly for e4m3fn; the quotients are x * 8
    x = np.array([[56.0, -1.5, 0.25], [3.0, -0.0, 7.0]], np.float32)
    q, s = tq.quant_tensor(_bits(x), "e4m3fn")
    assert s == np.float32(0.125)
    # 56*8 = 448 -> 0x7E; -12 = -1.5 * 2^3 -> E 10, M 4 -> 0xD4; 2 -> E 8 -> 0x40;
    # 24 = 1.5 * 2^4 -> E 11, M 4 -> 0x5C; -0 -> 0x80; 56 = 1.75 * 2^5 -> E 12, M 6 -> 0x66
    assert q.tolist() == [[0x7E, 0xD4, 0x40], [0x5C, 0x80, 0x66]]
    # e5m2: amax = 57344 * 2^-10 = 56 -> s = 2^-10; quotients x * 1024
    q5, s5 = tq.quant_tensor(_bits(x), "e5m2")
    assert s5 == np.float32(2.0 ** -10)
    assert q5[0, 0] == 0x7B  # amax -> largest finite e5m2


def test_hand_codes_e5m2():
    # 1.5 * 1024 = 1536 = 1.5 * 2^10 -> E = 25, M = 2 -> (25 << 2) | 2 = 0x66, negative -> 0xE6
    # 0.25 * 1024 = 256 = 2^8 -> E = 23, M = 0 -> 0x5C ; 3 * 1024 = 1.5 * 2^11 -> E = 26, M = 2 -> 0x6A
    x = np.array([56.0, -1.5, 0.25, 3.0], np.float32)
    q, _ = tq.quant_tensor(_bits(x), "e5m2")
    assert q.tolist() == [0x7B, 0xE6, 0x5C, 0x6A]


def test_worked_subnormal_scale_saturates_e5m2():
    # amax = 2^-133, the smallest positive bf16 (bits 0x0001). amax / 57344 = (8/7) * 2^-149
    # lies between the fp32 subnormals 2^-149 and 2^-148, nearer the first: s = 2^-149.
    # The quotient amax / s = 2^16 = 65536 is above 57344 and saturates to 0x7B (0xFB for
    # -amax); half of amax gives 2^15 = 32768 = 1.0 * 2^15 -> E = 30, M = 0 -> 0x78.
    bits = np.array([0x0001, 0x8001, 0x0000, 0x8000], np.uint16)
    q, s = tq.quant_tensor(bits, "e5m2")
    assert np.float32(s).view(np.uint32) == 1  # 2^-149
    assert q.tolist() == [0x7B, 0xFB, 0x00, 0x80]
    assert e5m2.decode(np.array([0x78], np.uint8))[0] == 32768.0
    # e4m3fn: amax / 448 = (2^16 / 448) * 2^-149 = 146.29 units of 2^-149 -> s = 146 * 2^-149,
    # quotient 65536 / 146 = 448.88 (below the 464 midpoint), saturating to 448 (0x7E)
    q4, s4 = tq.quant_tensor(bits, "e4m3fn")
    assert np.float32(s4).view(np.uint32) == 146
    assert q4.tolist() == [0x7E, 0xFE, 0x00, 0x80]


@pytest.mark.parametrize("fmt,fmax,rel", [("e4m3fn", 448.0, 2.0 ** -4), ("e5m2", 57344.0, 2.0 ** -3)])
def test_invariants(fmt, fmax, rel):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((37, 91)).astype(np.float32) * np.float32(3.0)
    bits = _bits(x)
    xf = quant.bf16_bits_to_f32(bits)
    q, s = tq.quant_tensor(bits, fmt)
    dec = (e4m3 if fmt == "e4m3fn" else e5m2).decode
    i = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
    assert abs(dec(q[i])) == fmax
    qn, sn = tq.quant_tensor(bits ^ np.uint16(0x8000), fmt)  # negate every element
    assert sn == s and np.array_equal(qn, q ^ np.uint8(0x80))
    q2, s2 = tq.quant_tensor(_bits(xf * np.float32(4.0)), fmt)  # exact 2^2 rescaling
    assert s2 == s * np.float32(4.0) and np.array_equal(q2, q)
    deq = tq.dequant_tensor(q, fmt, s).astype(np.float64)
    normal = np.abs(xf) >= (2.0 ** -6 if fmt == "e4m3fn" else 2.0 ** -14) * s
    err = np.abs(deq - xf)[normal] / np.abs(xf)[normal]
    assert err.max() <= rel * (1 + 1e-6)


def test_zero_tensor_and_rejection():
    z = np.array([[0, 0x8000, 0]], np.uint16)
    for fmt in ("e4m3fn", "e5m2"):
        q, s = tq.quant_tensor(z, fmt)
        assert s == 0 and q.tolist() == [[0, 0x80, 0]]
        with pytest.raises(ValueError):
            tq.quant_tensor(np.array([0x7F80], np.uint16), fmt)


def test_dequant_exact_products():
    rng = np.random.default_rng(3)
    s = np.float32(rng.random() * 0.01)
    for fmt, mod, n in (("e4m3fn", e4m3, 0x7F), ("e5m2", e5m2, 0x7C)):
        codes = np.arange(n, dtype=np.uint8)
        codes = np.concatenate([codes, codes | 0x80])
        got = tq.dequant_tensor(codes, fmt, s)
        exact = mod.decode(codes) * float(s)  # float64 holds the product exactly (<= 28 bits)
        assert np.array_equal(got, exact.astype(np.float32))
