"""The oracle's pins catch plausible mistakes: each test plants one mistake in the
oracle (on the CPU, through monkeypatch) and checks that a pin fails.
"""

import mpmath
import numpy as np
import pytest

import oracle.act as act_mod
import oracle.e4m3 as e4m3_mod
import oracle.e5m2 as e5m2_mod
import oracle.tensor_quant as tq_mod
import oracle.linear as linear_mod
import oracle.quant as quant_mod
import oracle.w8a16 as w8a16_mod
from tests import test_oracle_act as ta
from tests import test_oracle_e4m3 as te
from tests import test_oracle_e5m2 as t5
from tests import test_oracle_tensor_quant as ttq
from tests import test_oracle_linear as tl
from tests import test_oracle_quant as tq
from tests import test_oracle_w8a16 as tw

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_round_half_up_is_caught(monkeypatch):
    def encode_half_up(values):
        # the same steps as the oracle's encode with ties rounded away from zero
        v = np.asarray(values, np.float32).astype(np.float64)
        neg = np.signbit(v)
        a = np.minimum(np.abs(v), 448.0)
        sub = np.floor(a * 512.0 + 0.5)
        safe = np.where(a >= 2.0 ** -6, a, 1.0)
        _, e = np.frexp(safe)
        e = e.astype(np.int64) - 1
        m = np.floor((safe / np.exp2(e.astype(np.float64)) - 1.0) * 8.0 + 0.5).astype(np.int64)
        e = np.where(m == 8, e + 1, e)
        m = np.where(m == 8, 0, m)
        code = np.where(a < 2.0 ** -6, sub.astype(np.int64), ((e + 7) << 3) | m)
        return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)

    monkeypatch.setattr(e4m3_mod, "encode", encode_half_up)
    _fails(te.test_encode_matches_brute_force_at_every_boundary)


def test_missing_saturation_is_caught(monkeypatch):
    real = e4m3_mod.encode

    def encode_no_clamp(values):
        v = np.asarray(values, np.float32)
        out = real(v)
        return np.where(np.abs(v) > 448, np.uint8(0x7F) | (out & 0x80), out).astype(np.uint8)

    monkeypatch.setattr(e4m3_mod, "encode", encode_no_clamp)
    _fails(te.test_saturation_and_ties)


def test_lost_sign_of_zero_is_caught(monkeypatch):
    real = e4m3_mod.encode
    monkeypatch.setattr(e4m3_mod, "encode", lambda v: np.where(real(v) == 0x80, 0, real(v)).astype(np.uint8))
    _fails(tq.test_zero_rows_and_signed_zero)


def test_int8_denominator_is_caught(monkeypatch):
    monkeypatch.setattr(quant_mod, "_F448", np.float32(127.0))
    _fails(tq.test_worked_rows, GOLDEN)


def test_multiply_by_reciprocal_is_caught(monkeypatch):
    # x * (1/s) instead of the correctly rounded x / s differs near rounding boundaries
    real_encode = e4m3_mod.encode

    def quant_recip(x_f32):
        x = np.asarray(x_f32, np.float32)
        s = quant_mod.row_scales(x)
        q = np.empty(x.shape, np.uint8)
        nz = s > 0
        r = (np.float32(1.0) / s[nz]).astype(np.float32)
        q[nz] = real_encode((x[nz] * r[:, None]).astype(np.float32))
        q[~nz] = np.signbit(x[~nz]).astype(np.uint8) << 7
        return q, s

    monkeypatch.setattr(quant_mod, "quant_rows_f32", quant_recip)
    _fails(tq.test_hard_quotients_match_torch)


def test_reversed_k_pairing_is_caught(monkeypatch):
    # a wrong operand index: activation k paired with weight k' = K - 1 - k
    def gemm_misindexed(qa, qw):
        d = e4m3_mod.decode
        return d(qa)[:, ::-1] @ d(qw).T
    monkeypatch.setattr(linear_mod, "gemm_exact", gemm_misindexed)
    _fails(tl.test_linear_matches_python_loops)


def test_dropped_bias_is_caught(monkeypatch):
    real = linear_mod.epilogue
    monkeypatch.setattr(linear_mod, "epilogue", lambda acc, sa, sw, b=None: real(acc, sa, sw, None))
    _fails(tl.test_zero_activation_gives_bias)


def test_scales_on_swapped_axes_are_caught(monkeypatch):
    def epilogue_swapped(acc, a_scale, w_scale, bias_bits=None):
        acc = np.asarray(acc, np.float64)
        return acc * np.resize(np.asarray(w_scale, np.float64), acc.shape[0])[:, None] * \
            np.resize(np.asarray(a_scale, np.float64), acc.shape[1])[None, :]
    monkeypatch.setattr(linear_mod, "epilogue", epilogue_swapped)
    _fails(tl.test_bias_none_and_scales_broadcast_along_the_right_axes)


def test_amax_without_abs_is_caught(monkeypatch):
    def row_scales_signed(x_f32):
        x = np.asarray(x_f32, np.float32)
        return (np.max(x, axis=1).astype(np.float32) / np.float32(448.0)).astype(np.float32)
    monkeypatch.setattr(quant_mod, "row_scales", row_scales_signed)
    _fails(tq.test_invariants)


# --- activation producers (oracle.act): mistakes planted in the exact evaluation


def _act_sample():
    rng = np.random.default_rng(11)
    pats = act_mod._finite_patterns()
    return np.sort(rng.choice(pats, 1500, replace=False)).astype(np.uint16)


def _act_planted(monkeypatch, kind, wrong):
    real = act_mod._act_mp
    monkeypatch.setattr(act_mod, "_act_mp", lambda x, k: wrong(x) if k == kind else real(x, k))
    pats = _act_sample()
    return pats, act_mod.act_bits_exact(pats, kind)


def test_gelu_erf_wrong_sign_is_caught(monkeypatch):
    pats, vals = _act_planted(monkeypatch, "gelu_erf", lambda x: x * mpmath.erfc(x / mpmath.sqrt(2)) / 2)
    _fails(ta.check_against_float64, "gelu_erf", pats, vals)


def test_gelu_tanh_wrong_constant_is_caught(monkeypatch):
    def wrong(x):
        u = mpmath.sqrt(2 / mpmath.pi) * (x + mpmath.mpf("0.0447") * x ** 3)
        return x / (1 + mpmath.exp(-2 * u))
    pats, vals = _act_planted(monkeypatch, "gelu_tanh", wrong)
    _fails(ta.check_against_float64, "gelu_tanh", pats, vals)


def test_silu_wrong_exponent_sign_is_caught(monkeypatch):
    pats, vals = _act_planted(monkeypatch, "silu", lambda x: x / (1 + mpmath.exp(x)))
    _fails(ta.check_against_float64, "silu", pats, vals)


def test_float64_evaluation_is_caught(monkeypatch):
    # evaluating in float64 instead of exactly loses the x^2 term that decides the ties
    def f64(x):
        v = float(x)
        return mpmath.mpf(0.5 * v * float(mpmath.erfc(-v / 2 ** 0.5)))
    pats, vals = _act_planted(monkeypatch, "gelu_erf", f64)
    pats = np.concatenate([pats, np.arange(1, 256, dtype=np.uint16)])  # the tiny inputs
    vals = act_mod.act_bits_exact(pats, "gelu_erf")
    _fails(ta.check_ties, "gelu_erf", pats, vals)


def test_bf16_ties_away_from_zero_are_caught(monkeypatch):
    real_floor = mpmath.floor

    def round_away(y):
        y = mpmath.mpf(y)
        if y == 0:
            return np.uint16(0)
        neg = y < 0
        a = -y if neg else y
        _, e = mpmath.frexp(a)
        qe = max(int(e) - 8, -133)
        f = real_floor(mpmath.ldexp(a, -qe) + mpmath.mpf(0.5))
        val = float(mpmath.ldexp(f, qe))
        bits = np.array([val], np.float32).view(np.uint32)[0] >> np.uint32(16)
        return np.uint16(bits | (0x8000 if neg else 0))
    monkeypatch.setattr(act_mod, "round_bf16", round_away)
    _fails(ta.test_round_bf16_matches_torch_on_float32_values)


def test_bf16_without_subnormals_is_caught(monkeypatch):
    real = act_mod.round_bf16

    def flush(y):
        if isinstance(y, float) and 0 < abs(y) < 2.0 ** -126:
            return np.uint16(0x8000 if y < 0 else 0)
        return real(y)
    monkeypatch.setattr(act_mod, "round_bf16", flush)
    _fails(ta.test_round_bf16_matches_torch_on_float32_values)


# --- the FP8 weight-only linear (oracle.w8a16)


def test_w8a16_reversed_k_is_caught(monkeypatch):
    def wrong(a_bits, qw, w_scale, bias_bits=None):
        a = quant_mod.bf16_bits_to_f32(np.asarray(a_bits, np.uint16)).astype(np.float64)
        out = (a[:, ::-1] @ e4m3_mod.decode(np.asarray(qw, np.uint8)).T) * np.asarray(w_scale, np.float64)[None, :]
        if bias_bits is not None:
            out = out + quant_mod.bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
        return out
    monkeypatch.setattr(w8a16_mod, "w8a16_ref", wrong)
    _fails(tw.test_matches_exact_rational_brute_force)


def test_w8a16_scale_on_the_token_axis_is_caught(monkeypatch):
    real = w8a16_mod.w8a16_ref

    def wrong(a_bits, qw, w_scale, bias_bits=None):
        base = real(a_bits, qw, np.ones_like(np.asarray(w_scale, np.float32)), bias_bits)
        return base * np.resize(np.asarray(w_scale, np.float64), base.shape[0])[:, None]
    monkeypatch.setattr(w8a16_mod, "w8a16_ref", wrong)
    _fails(tw.test_scales_act_per_output_channel)


def test_w8a16_dropped_scale_is_caught(monkeypatch):
    real = w8a16_mod.w8a16_ref
    monkeypatch.setattr(w8a16_mod, "w8a16_ref",
                        lambda a, qw, sw, b=None: real(a, qw, np.ones_like(np.asarray(sw, np.float32)), b))
    _fails(tw.test_equals_w8a8_where_the_activation_quant_is_the_identity)


# --- e5m2 codes and the per-tensor quantiser


def test_e5m2_wrong_bias_is_caught(monkeypatch):
    real = e5m2_mod.decode
    monkeypatch.setattr(e5m2_mod, "decode", lambda c: real(c) * 0.5)  # as if the exponent bias were 16
    _fails(t5.test_decode_landmarks, GOLDEN)


def test_e5m2_half_up_is_caught(monkeypatch):
    def encode_half_up(values):
        v = np.asarray(values, np.float32).astype(np.float64)
        neg = np.signbit(v)
        a = np.minimum(np.abs(v), 57344.0)
        sub = np.floor(a * 2.0 ** 16 + 0.5)
        safe = np.where(a >= 2.0 ** -14, a, 1.0)
        _, e = np.frexp(safe)
        e = e.astype(np.int64) - 1
        m = np.floor((safe / np.exp2(e.astype(np.float64)) - 1.0) * 4.0 + 0.5).astype(np.int64)
        e = np.where(m == 4, e + 1, e)
        m = np.where(m == 4, 0, m)
        code = np.where(a < 2.0 ** -14, sub.astype(np.int64), ((e + 15) << 2) | m)
        return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)
    monkeypatch.setattr(e5m2_mod, "encode", encode_half_up)
    _fails(t5.test_encode_matches_brute_force_at_every_boundary)


def test_e5m2_missing_saturation_is_caught(monkeypatch):
    # without the clamp a quotient of 65536 (the smallest bf16 amax over its rounded-down
    # subnormal scale) would encode as 0x7C, the infinity code
    real = e5m2_mod.encode
    monkeypatch.setattr(e5m2_mod, "E5M2_MAX", np.inf)
    assert real(np.array([65536.0], np.float32))[0] == 0x7C
    _fails(ttq.test_worked_subnormal_scale_saturates_e5m2)


def test_per_row_scale_in_the_tensor_quantiser_is_caught(monkeypatch):
    def per_row(x_bits, fmt):
        q, s = quant_mod.quant_rows(np.atleast_2d(np.asarray(x_bits, np.uint16)))
        return q.reshape(np.shape(x_bits)), s[0]
    monkeypatch.setattr(tq_mod, "quant_tensor", per_row)
    _fails(ttq.test_worked_tensor_power_of_two_scale)
