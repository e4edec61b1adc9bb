"""Per-tensor FP8 quantisation and dequantisation (the state-dict converter's one-scale-per-tensor method).

Test infrastructure: part of the CPU oracle (see the package docstring for who
may import it).

The QuantizeFP8Format page (runcomfy.com, "Quantize Model to FP8 Format") converts
every tensor of a state dict to float8_e4m3fn or float8_e5m2 by scaling it and gives
no formula. The Stable Diffusion 3.5 FP8 page (dn008.com.cn,
section on FP8, steps 1-4) gives the steps: the largest magnitude of the tensor,
a scale from it, x / scale rounded to the 8-bit format, and x_q * scale back in fp32
at inference. The plainest reading, one scale per tensor:

    s = fl32(amax / fmax)          fmax = 448 (e4m3fn) or 57344 (e5m2)
    q = RNE_sat(fl32(x / s))       (all-zero tensor: s = 0, signed-zero codes)
    x' = fl32(dec(q) * s)          (dequantisation, fp32)

with the same precision rules as the per-token quantiser (oracle.quant): fp32 scale,
correctly rounded fp32 quotient, round to nearest even, saturating.
"""

import numpy as np

from . import e4m3, e5m2
from .quant import bf16_bits_to_f32

FORMATS = {"e4m3fn": (e4m3, np.float32(448.0)), "e5m2": (e5m2, np.float32(57344.0))}


def tensor_scale(x_f32, fmt):
    mod, fmax = FORMATS[fmt]
    x = np.asarray(x_f32, np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    return np.float32(amax / fmax)


def quant_tensor(x_bits, fmt):
    """Per-tensor quantisation of bf16 bits (any shape) -> (codes uint8 of the same shape, scale float32)."""
    mod, _ = FORMATS[fmt]
    x = bf16_bits_to_f32(np.asarray(x_bits, np.uint16))
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    s = tensor_scale(x, fmt)
    if s == 0:
        return (np.signbit(x).astype(np.uint8) << 7), s
    q = x / s  # float32 / float32 -> correctly rounded float32
    assert q.dtype == np.float32
    return mod.encode(q), s


def dequant_tensor(codes, fmt, scale):
    """x' = fl32(dec(q) * s), float32, same shape as the codes."""
    mod, _ = FORMATS[fmt]
    return (mod.decode(np.asarray(codes, np.uint8)).astype(np.float32) * np.float32(scale)).astype(np.float32)
