"""OCP FP8 E5M2 codes, written from the format definition.

Test infrastructure: part of the CPU oracle (see the package docstring for who
may import it).

The QuantizeFP8Format page (runcomfy.com, "Quantize Model to FP8 Format", input
parameters) offers float8_e5m2 beside float8_e4m3fn, e5m2 being its default; the
Stable Diffusion 3.5 FP8 page (dn008.com.cn, section on FP8 formats) names E5M2 as
5 exponent and 2 mantissa bits. The bit-level meaning is the OCP 8-bit floating
point specification's E5M2 encoding (IEEE-like):

  byte = S EEEEE MM, exponent bias 15
  E == 0          value = (-1)^S * M * 2^-16           (zero and subnormals)
  1 <= E <= 30    value = (-1)^S * (1 + M/4) * 2^(E-15)
  E == 31         infinity (M == 0) or NaN (M != 0)
  largest finite magnitude 57344 (0x7B); smallest subnormal 2^-16; smallest normal 2^-14

The QuantizeFP8Format page calls e5m2 the more precise choice; it has the wider
range and the coarser steps (2 mantissa bits against 3), so that claim is not used.
"""

import numpy as np

E5M2_MAX = 57344.0


def decode(codes):
    """Real value of each e5m2 byte, as float64 (+-inf for 0x7C / 0xFC, NaN for the rest of E = 31)."""
    c = np.asarray(codes).astype(np.int64)
    if c.size and (c.min() < 0 or c.max() > 255):
        raise ValueError("e5m2 codes are bytes 0..255")
    sign = (c >> 7) & 1
    exp = (c >> 2) & 0x1F
    man = c & 0x3
    sub = man.astype(np.float64) * 2.0 ** -16
    norm = (1.0 + man.astype(np.float64) / 4.0) * np.exp2(exp.astype(np.float64) - 15.0)
    mag = np.where(exp == 0, sub, norm)
    mag = np.where((exp == 31) & (man == 0), np.inf, mag)
    mag = np.where((exp == 31) & (man != 0), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def encode(values):
    """Round each finite float32 value to the nearest e5m2 code (RNE, saturating at +-57344).

    As for e4m3fn: clamp to the largest finite magnitude, then round to nearest with
    ties to the even mantissa (also among subnormals: 2^-17 -> 0, 3 * 2^-17 -> 2^-15);
    the sign is kept (-0.0 and negative values that round to zero give 0x80).
    """
    v32 = np.asarray(values, dtype=np.float32)
    if not np.all(np.isfinite(v32)):
        raise ValueError("e5m2 encode is defined for finite inputs only")
    v = v32.astype(np.float64)
    negative = np.signbit(v)
    a = np.minimum(np.abs(v), E5M2_MAX)
    # subnormal grid M * 2^-16 (M = 0..3); M = 4 is the smallest normal, code 0x04
    sub_code = np.rint(a * 2.0 ** 16)
    safe = np.where(a >= 2.0 ** -14, a, 1.0)
    _, e = np.frexp(safe)
    e = e.astype(np.int64) - 1
    mant = np.rint((safe / np.exp2(e.astype(np.float64)) - 1.0) * 4.0).astype(np.int64)
    carry = mant == 4
    e = np.where(carry, e + 1, e)
    mant = np.where(carry, 0, mant)
    norm_code = ((e + 15) << 2) | mant
    code = np.where(a < 2.0 ** -14, sub_code.astype(np.int64), norm_code)
    code = code | (negative.astype(np.int64) << 7)
    return code.astype(np.uint8)


def finite_values():
    """The 124 non-negative finite e5m2 values in code order 0x00..0x7B (float64)."""
    return decode(np.arange(0x7C, dtype=np.uint8))
