"""Per-row FP8 quantisation: dynamic per-token activations and per-channel weights.

Test infrastructure: part of the CPU oracle (see the package docstring for who
may import it).

Steps, in the order the pages give them for post-training quantisation (Stable
Diffusion 3.5 FP8 ComfyUI page, dn008.com.cn, section on FP8, steps 1-3): take
the largest magnitude of the tensor slice, divide it by the format's largest
value to get the scale, then divide every element by the scale and round it to
the 8-bit format. The HunyuanVideo1.5 retrospective (aigcage.com, section 2 and
section 3.1) fixes the granularity: one scale per token (row of the activation,
computed at run time) and one per output channel (row of the nn.Linear weight
[N, K], computed ahead of time). The two are the same per-row operation.

Readings where the pages are silent or wrong:
  * the denominator is 448, the largest finite e4m3fn value (the dn008 page's
    2^7 - 1 = 127 is the INT8 constant);
  * "round" means round to the nearest e4m3fn value, ties to even, saturating;
  * the scale is float32, s = fl32(amax / 448), and each quotient is the
    correctly rounded float32 x / s, which is then rounded to e4m3fn (this is
    the precision the kernel decides codes in, so both sides decide in it);
  * an all-zero row gets s = 0 and signed-zero codes (0x00 / 0x80), no division.
"""

import numpy as np

from . import e4m3

_F448 = np.float32(448.0)


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns (uint16) to their exact float32 values (bits << 16)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def row_scales(x_f32):
    """s[r] = fl32(max_k |x[r, k]| / 448) for a float32 matrix [R, C]."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    return (amax.astype(np.float32) / _F448).astype(np.float32)


def quant_rows_f32(x_f32):
    """Quantise each row of a finite float32 matrix [R, C] -> (codes uint8 [R, C], scales float32 [R])."""
    x = np.asarray(x_f32, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("quant_rows expects a 2-D [rows, cols] matrix")
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    s = row_scales(x)
    codes = np.empty(x.shape, dtype=np.uint8)
    zero = s == 0
    if np.any(zero):
        # amax == 0: every element is +-0; keep the sign, no division
        codes[zero] = (np.signbit(x[zero]).astype(np.uint8) << 7)
    nz = ~zero
    if np.any(nz):
        quotient = x[nz] / s[nz][:, None]  # float32 / float32 -> correctly rounded float32
        assert quotient.dtype == np.float32
        codes[nz] = e4m3.encode(quotient)
    return codes, s


def quant_rows(x_bits):
    """Dynamic per-token quantisation of a bf16 matrix given as uint16 bits [R, C]."""
    return quant_rows_f32(bf16_bits_to_f32(x_bits))


def quant_weights_per_channel(w_bits):
    """Per-output-channel weight quantisation of W bf16 [N, K]: the same per-row operation."""
    return quant_rows(w_bits)
