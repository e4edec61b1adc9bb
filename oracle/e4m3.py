"""OCP FP8 E4M3 ("e4m3fn") codes, written from the format definition.

Test infrastructure: part of the CPU oracle (see the package docstring for who
may import it).

The pages fix the format only as "4 exponent bits + 3 mantissa bits" and name
torch's ``float8_e4m3fn`` dtype (Stable Diffusion 3.5 FP8 ComfyUI page,
dn008.com.cn, section on FP8 formats; HunyuanVideo1.5 retrospective section 3.5
for the float8_e4m3fn input contract). The bit-level meaning is the OCP 8-bit
floating point specification's E4M3 encoding:

  byte = S EEEE MMM, exponent bias 7
  E == 0          value = (-1)^S * M * 2^-9             (zero and subnormals)
  E >= 1          value = (-1)^S * (1 + M/8) * 2^(E-7)
  E == 15, M == 7 NaN (0x7F, 0xFF); there is no infinity
  largest finite magnitude 448 (0x7E); smallest subnormal 2^-9; smallest normal 2^-6

The pages' own range claim for E4M3 (about 1e-6 .. 1e8) is wrong and is not used.
"""

import numpy as np

E4M3_MAX = 448.0


def _decode_formula(c):
    """The closed form above, evaluated elementwise on int64 codes 0..255."""
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = man.astype(np.float64) * 2.0 ** -9
    # 2^(E-7) for E in 1..15; E == 0 lanes are replaced by the subnormal value below
    norm = (1.0 + man.astype(np.float64) / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    mag = np.where(exp == 0, sub, norm)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# The closed form evaluated once on all 256 codes; decode() looks values up here, so
# decoding a large matrix costs one indexing pass rather than the formula per element.
_VALUES = _decode_formula(np.arange(256, dtype=np.int64))


def decode(codes):
    """Real value of each e4m3fn byte, as float64 (NaN for 0x7F / 0xFF, -0.0 for 0x80)."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        c = c.astype(np.int64)
        if c.size and (c.min() < 0 or c.max() > 255):
            raise ValueError("e4m3fn codes are bytes 0..255")
    return _VALUES[c]


def encode(values):
    """Round each finite float32 value to the nearest e4m3fn code (RNE, saturating).

    Saturation: magnitudes above 448 become 448 (clamp first; rounding the
    clamped value to nearest-even is the same as saturating after rounding).
    Ties go to the even mantissa, also in the subnormal range (2^-10 -> 0,
    3*2^-10 -> 2*2^-9). The sign is kept, so -0.0 and negative values that
    round to zero give 0x80. NaN and infinity are outside the contract.
    """
    v32 = np.asarray(values, dtype=np.float32)
    if not np.all(np.isfinite(v32)):
        raise ValueError("e4m3fn encode is defined for finite inputs only")
    v = v32.astype(np.float64)  # exact
    negative = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)

    # Subnormal range a < 2^-6: the grid is M * 2^-9, M = 0..7; M = 8 is the
    # smallest normal (code 0x08), so the rounded integer is the code itself.
    sub_code = np.rint(a * 2.0 ** 9)  # numpy rint rounds half to even

    # Normal range: a = f * 2^e with f in [1, 2); the mantissa is (f - 1) * 8
    # rounded to nearest even; a carry out of the mantissa bumps the exponent.
    safe = np.where(a >= 2.0 ** -6, a, 1.0)
    frac, e = np.frexp(safe)  # safe = frac * 2^e, frac in [0.5, 1)
    e = e.astype(np.int64) - 1
    mant = np.rint((safe / np.exp2(e.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    e = np.where(carry, e + 1, e)
    mant = np.where(carry, 0, mant)
    norm_code = ((e + 7) << 3) | mant

    code = np.where(a < 2.0 ** -6, sub_code.astype(np.int64), norm_code)
    code = code | (negative.astype(np.int64) << 7)
    return code.astype(np.uint8)


def finite_values():
    """The 127 non-negative finite e4m3fn values in code order 0x00..0x7E (float64)."""
    return decode(np.arange(0x7F, dtype=np.uint8))
