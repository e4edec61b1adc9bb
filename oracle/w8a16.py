"""FP8 weight-only linear (W8A16): bf16 activation times an e4m3fn weight with per-channel scales.

Test infrastructure: part of the CPU oracle (see the package docstring for who
may import it).

The LongCat avatar comparison page (longcat-avatar-compare.pages.dev, speed
overview table) measures an FP8 weight-only pipeline beside the W4A4 one:
the weights are stored as FP8 with scales and the activations stay in 16-bit. The
page gives no formula; the plainest reading, with the per-output-channel weight
quantisation of the HunyuanVideo1.5 retrospective (aigcage.com, section 2) and
nn.Linear's [N, K] layout, is

    out[m, n] = sum_k a[m, k] * (dec(qw[n, k]) * sw[n]) + bias[n]
              = sw[n] * sum_k a[m, k] * dec(qw[n, k]) + bias[n]

(the scale is constant along k, so it may be applied after the sum). The
activation is not quantised. The reference is evaluated in float64 and left
unrounded: every bf16 value and every e4m3fn value is exact in float64, each
product is exact (at most 12 significant bits), and the float64 sum carries a
relative error of at most about K * 2^-53 of sum |a * dec(qw)|, far below what
the tests resolve.


The weight codes may also be e5m2 (the default format of the QuantizeFP8Format
state-dict converter, runcomfy.com, input parameters), with a per-tensor scale
repeated over the output channels; every finite e5m2 value is also exact in float64.
"""

import numpy as np

from . import e4m3, e5m2
from .quant import bf16_bits_to_f32

_DECODE = {"e4m3fn": e4m3.decode, "e5m2": e5m2.decode}


def dequant_weight(qw, w_scale, fmt="e4m3fn"):
    """The weight the layer represents: dec(qw[n, k]) * sw[n], float64 [N, K]."""
    return _DECODE[fmt](np.asarray(qw, np.uint8)) * np.asarray(w_scale, np.float32).astype(np.float64)[:, None]


def w8a16_ref(a_bits, qw, w_scale, bias_bits=None, fmt="e4m3fn"):
    """out [M, N] float64 for a bf16 activation (uint16 bits [M, K]) and FP8 weight codes [N, K]."""
    a = bf16_bits_to_f32(np.asarray(a_bits, np.uint16)).astype(np.float64)
    qw = np.asarray(qw, np.uint8)
    if a.ndim != 2 or qw.ndim != 2 or a.shape[1] != qw.shape[1]:
        raise ValueError("w8a16_ref expects a [M, K] and qw [N, K]")
    out = (a @ _DECODE[fmt](qw).T) * np.asarray(w_scale, np.float32).astype(np.float64)[None, :]
    if bias_bits is not None:
        out = out + bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return out
