"""Activation producers that emit FP8 directly: GELU / SiLU followed by per-token quant.

Test infrastructure: part of the CPU oracle (see the package docstring for who
may import it).

The HunyuanVideo1.5 retrospective (aigcage.com, section 3, item 5 "producer
fusion") describes the step upstream of the FFN-down linear: the plain path has
GELU or SiLU write a bf16 tensor, quantises that tensor per token to FP8 and then
runs the FP8 GEMM; the fused producer hands the (fp8 codes, per-token scale) pair
straight to the FP8 linear. The fusion removes memory traffic, not arithmetic, so
its result is defined as the plain path's:

    y = bf16_RNE(act(x))           for every bf16 element x of the row
    (codes, scale) = quant_rows(y)  (the per-token quantiser of oracle.quant)

Readings where the page is silent:
  * it names "GELU/SiLU" and no formula. Three textbook functions are provided:
      gelu_erf   x * Phi(x) = x/2 * erfc(-x / sqrt 2)          (exact GELU)
      gelu_tanh  x/2 * (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))  (its tanh form)
      silu       x * sigmoid(x) = x / (1 + exp(-x))
    with the real-number constants exactly as written;
  * "GELU produces bf16" is read as the correctly rounded bf16 of the exact
    function value (round to nearest, ties to even), not any one library's fp32
    approximation;
  * non-finite inputs are outside the contract (their table entries are not
    defined here).

Because x is bf16, act is a map from 2^16 bit patterns to 2^16 bit patterns. The
oracle evaluates it at 300-bit precision (mpmath) and rounds that exactly. Float64
is not enough to define the rounding: for |x| < 2^-125, x/2 can fall exactly
halfway between two bf16 values and the function's tiny x^2 term (lost in
float64) decides the direction.
"""

import functools

import mpmath
import numpy as np

from .quant import quant_rows

ACTS = ("gelu_erf", "gelu_tanh", "silu")

_PREC = 300  # bits; every finite bf16 input's value is decided far inside this


def _act_mp(x, kind):
    """act(x) for an mpmath number x at the context precision."""
    if kind == "gelu_erf":
        return x * mpmath.erfc(-x / mpmath.sqrt(2)) / 2
    if kind == "gelu_tanh":
        u = mpmath.sqrt(2 / mpmath.pi) * (x + mpmath.mpf(44715) / 10 ** 6 * x ** 3)
        # 1 + tanh(u) = 2 / (1 + exp(-2u)); the same value without cancellation for u << 0
        return x / (1 + mpmath.exp(-2 * u))
    if kind == "silu":
        return x / (1 + mpmath.exp(-x))
    raise ValueError(f"unknown activation {kind!r}")


def round_bf16(y):
    """Round a real number (mpmath or float) to the nearest bf16, ties to even; returns uint16 bits.

    bf16 has 8 significant bits and the float32 exponent range, with subnormals of
    quantum 2^-133. |y| large enough to overflow does not arise from these
    functions (|act(x)| <= |x|).
    """
    if isinstance(y, float) and y == 0.0:
        return np.uint16(0x8000 if np.signbit(y) else 0)
    y = mpmath.mpf(y)
    if y == 0:
        return np.uint16(0)
    neg = y < 0
    a = -y if neg else y
    _, e = mpmath.frexp(a)  # a = m * 2^e, m in [0.5, 1): a in [2^(e-1), 2^e)
    quantum_exp = max(int(e) - 8, -133)
    q = mpmath.ldexp(a, -quantum_exp)  # a / quantum, a real number
    f = mpmath.floor(q)
    d = q - f
    if d > 0.5 or (d == 0.5 and int(f) % 2 == 1):
        f += 1
    val = float(mpmath.ldexp(f, quantum_exp))  # an exact bf16 value
    bits = np.array([val], np.float32).view(np.uint32)[0] >> np.uint32(16)
    return np.uint16(bits | (0x8000 if neg else 0))


def _finite_patterns():
    pat = np.arange(1 << 16, dtype=np.uint32)
    return pat[((pat >> 7) & 0xFF) != 0xFF]


def act_bits_exact(patterns, kind):
    """bf16_RNE(act(x)) for the given finite bf16 bit patterns, evaluated one by one."""
    if kind not in ACTS:
        raise ValueError(f"unknown activation {kind!r}")
    pats = np.asarray(patterns, np.uint16).astype(np.uint32)
    xs = (pats << np.uint32(16)).view(np.float32)
    out = np.empty(len(pats), np.uint16)
    with mpmath.workprec(_PREC):
        for i, (p, x) in enumerate(zip(pats, xs)):
            if x == 0:
                out[i] = np.uint16(p)  # act(+-0) = +-0 for all three
                continue
            out[i] = round_bf16(_act_mp(mpmath.mpf(float(x)), kind))
    return out


@functools.lru_cache(maxsize=None)
def table(kind):
    """(patterns, results): every finite bf16 input pattern and bf16_RNE(act(x)) as uint16."""
    pats = _finite_patterns().astype(np.uint16)
    return pats, act_bits_exact(pats, kind)


@functools.lru_cache(maxsize=None)
def full_table(kind):
    """A 65536-entry lookup indexed by the input pattern; non-finite inputs map to 0xFFFF."""
    pats, vals = table(kind)
    t = np.full(1 << 16, 0xFFFF, np.uint16)
    t[pats] = vals
    return t


def act_bf16_bits(x_bits, kind):
    """bf16_RNE(act(x)) for an array of finite bf16 bit patterns."""
    x = np.asarray(x_bits, np.uint16)
    exp = (x >> 7) & 0xFF
    if np.any(exp == 0xFF):
        raise ValueError("inputs must be finite")
    return full_table(kind)[x]


def act_quant_rows(x_bits, kind):
    """The fused producer's result: per-token quant of bf16_RNE(act(x)) -> (codes [R, C], scales [R])."""
    return quant_rows(act_bf16_bits(x_bits, kind))
