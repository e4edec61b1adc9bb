"""Pins for oracle.act: GELU / SiLU rounded to bf16, then per-token FP8.

The oracle evaluates each activation at 300-bit precision and rounds exactly. It is
pinned here against things fixed outside it: torch's float32 -> bf16 conversion
(round to nearest even) for the rounding, float64 evaluations built on scipy's and
torch's special-function routines (a different implementation of erfc / the
logistic function), textbook values, and the Taylor series at the origin, which
predicts exactly which inputs float64 cannot decide and which way they round.
"""

import mpmath
import numpy as np
import pytest
import scipy.special as sp
import torch

from oracle import act, quant

TINY = 2.0 ** -125


def _x(pats):
    return (np.asarray(pats, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _f64(kind, x):
    """act(x) in float64 from library special functions (scipy's erfc and logistic)."""
    x = np.asarray(x, np.float64)
    if kind == "gelu_erf":
        return 0.5 * x * sp.erfc(-x / np.sqrt(2.0))
    if kind == "gelu_tanh":
        return x * sp.expit(2.0 * np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3))
    return x * sp.expit(x)


def _round_all(y):
    return np.array([act.round_bf16(float(v)) for v in y], np.uint16)


def _tie_inputs(pats):
    """|x| < 2^-125 and x an odd multiple of 2^-133: x / 2 lies halfway between two bf16 values."""
    x = _x(pats).astype(np.float64)
    k = np.round(np.abs(x) / 2.0 ** -133)
    return (np.abs(x) < TINY) & (x != 0) & (k % 2 == 1)


def check_against_float64(kind, pats, vals):
    """Outside the tie inputs, the exact table equals the rounded float64 library value."""
    x = _x(pats)
    ties = _tie_inputs(pats)
    r = _round_all(_f64(kind, x[~ties]))
    bad = np.nonzero(r != vals[~ties])[0]
    assert len(bad) == 0, f"{kind}: {len(bad)} disagreements, first x = {x[~ties][bad[:5]]}"


def check_ties(kind, pats, vals):
    """act(x) = x/2 + c x^2 + O(x^3) with c > 0: at a tie, the x^2 term rounds x/2 toward +inf."""
    ties = _tie_inputs(pats)
    assert np.any(ties)
    half = _x(pats)[ties].astype(np.float64) / 2  # exact midpoints
    with mpmath.workprec(600):
        up = np.array([act.round_bf16(mpmath.mpf(h) + mpmath.ldexp(1, -500)) for h in half], np.uint16)
    assert np.array_equal(vals[ties], up)
    # and plain round-half-even of x/2 (what float64 gives) differs on about half of them
    even = _round_all(half)
    assert 0 < np.sum(even != up) < len(half)


@pytest.mark.parametrize("kind", act.ACTS)
def test_table_matches_float64_library_values(kind):
    pats, vals = act.table(kind)
    assert len(pats) == (1 << 16) - 256  # every finite bf16 pattern
    check_against_float64(kind, pats, vals)


@pytest.mark.parametrize("kind", act.ACTS)
def test_tie_inputs_round_toward_plus_infinity(kind):
    pats, vals = act.table(kind)
    # odd multiples of 2^-133 below 2^-125: 64 subnormal and 64 exponent-1 codes per sign
    assert int(np.sum(_tie_inputs(pats))) == 256
    check_ties(kind, pats, vals)


@pytest.mark.parametrize("kind", act.ACTS)
def test_float64_decides_every_other_input(kind):
    # every non-tie value sits well away from a bf16 rounding midpoint, relative to its
    # size: any evaluation with relative error below 1e-9 rounds to the table
    pats, vals = act.table(kind)
    x = _x(pats)
    keep = ~_tie_inputs(pats) & (x != 0)
    y = np.abs(_f64(kind, x[keep]))
    y = y[y > 2.0 ** -134]  # below half the smallest subnormal: rounds to zero with room
    e = np.floor(np.log2(y))
    quantum = 2.0 ** np.maximum(e - 7, -133)
    frac = y / quantum
    margin = np.abs(frac - np.floor(frac) - 0.5) * quantum / y
    assert margin.min() > 1e-9


def test_torch_double_agrees_in_the_core():
    # torch's own float64 GELU / tanh-GELU / SiLU, where their formulas do not cancel
    pats, _ = act.table("silu")
    x = _x(pats)
    core = (np.abs(x) <= 3.0) & ~_tie_inputs(pats)
    xt = torch.from_numpy(x[core].astype(np.float64))
    refs = {
        "gelu_erf": torch.nn.functional.gelu(xt).numpy(),
        "gelu_tanh": torch.nn.functional.gelu(xt, approximate="tanh").numpy(),
        "silu": torch.nn.functional.silu(xt).numpy(),
    }
    for kind, y in refs.items():
        tab = act.full_table(kind)[pats[core]]
        assert np.array_equal(_round_all(y), tab), kind


def test_textbook_values():
    # Phi(1) = 0.8413447460685429..., Phi(-1) = 0.1586552539314571...; sigmoid(1) = 0.7310585786300049...
    cases = [
        ("gelu_erf", 1.0, 0.8413447460685429),
        ("gelu_erf", -1.0, -0.15865525393145707),
        ("gelu_erf", 2.0, 1.9544997361036416),
        ("silu", 1.0, 0.7310585786300049),
        ("silu", -2.0, -0.23840584404423515),
        ("gelu_tanh", 1.0, 0.8411919906082768),
    ]
    for kind, x, y in cases:
        xb = np.array([x], np.float32).view(np.uint32)[0] >> 16
        assert act.act_bf16_bits(np.array([xb], np.uint16), kind)[0] == act.round_bf16(y), (kind, x)
    # far tails: GELU(x) = x for large x; SiLU keeps a nonzero bf16 tail down to about -88
    big = np.array([0x4200], np.uint16)  # 32.0
    for kind in act.ACTS:
        assert act.act_bf16_bits(big, kind)[0] == 0x4200
    neg80 = np.array([0xC2A0], np.uint16)  # -80.0
    assert act.act_bf16_bits(neg80, "silu")[0] != 0x8000
    assert act.act_bf16_bits(neg80, "gelu_erf")[0] == 0x8000  # -80 Phi(-80) underflows bf16: -0


def test_signed_zero_and_rejections():
    z = np.array([0x0000, 0x8000], np.uint16)
    for kind in act.ACTS:
        assert np.array_equal(act.act_bf16_bits(z, kind), z)
        with pytest.raises(ValueError):
            act.act_bf16_bits(np.array([0x7F80], np.uint16), kind)
    with pytest.raises(ValueError):
        act.table("relu")


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]
    # exact midpoints and their neighbours, normal and subnormal, both signs
    mids = (rng.integers(0, 1 << 16, 3000).astype(np.uint32) << 16) | 0x8000
    mids = mids[((mids >> 23) & 0xFF) < 0xFE]
    bits = np.concatenate([bits, mids, mids + 1, mids - 1, np.arange(0, 1 << 17, 97, dtype=np.uint32)])
    vals = bits.view(np.float32)
    ours = _round_all(vals.astype(np.float64))
    theirs = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_round_bf16_below_float64_resolution():
    one = mpmath.mpf(1)
    mid = one + mpmath.ldexp(1, -8)  # halfway between 1 and 1 + 2^-7
    with mpmath.workprec(400):
        assert act.round_bf16(mid) == 0x3F80  # tie -> even (1.0)
        assert act.round_bf16(mid + mpmath.ldexp(1, -350)) == 0x3F81
        assert act.round_bf16(mid - mpmath.ldexp(1, -350)) == 0x3F80
        odd_mid = one + 3 * mpmath.ldexp(1, -8)  # halfway between 1 + 2^-7 (odd) and 1 + 2^-6
        assert act.round_bf16(odd_mid) == 0x3F82
        assert act.round_bf16(-odd_mid) == 0xBF82
        sub_mid = mpmath.ldexp(1, -134)  # halfway between 0 and the smallest subnormal
        assert act.round_bf16(sub_mid) == 0x0000
        assert act.round_bf16(sub_mid + mpmath.ldexp(1, -380)) == 0x0001
    assert act.round_bf16(-0.0) == 0x8000


def test_act_quant_rows_worked_row():
    # SiLU of [2, -1, 0.5, -0] by hand: 1.7615941559557649, -0.2689414213699951,
    # 0.3112296656009784, -0 -> bf16 1.7578125 (0x3FE1), -0.26953125 (0xBE8A),
    # 0.310546875 (0x3E9F), -0; amax 1.7578125 -> s = fl32(1.7578125 / 448)
    x = np.array([[0x4000, 0xBF80, 0x3F00, 0x8000]], np.uint16)
    y = act.act_bf16_bits(x, "silu")
    assert y.tolist() == [[0x3FE1, 0xBE8A, 0x3E9F, 0x8000]]
    q, s = act.act_quant_rows(x, "silu")
    assert s[0] == np.float32(1.7578125) / np.float32(448.0)
    assert q[0, 0] == 0x7E  # the row maximum maps to 448
    q2, s2 = quant.quant_rows(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
