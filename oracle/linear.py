"""FP8 W8A8 linear: exact FP8 product, then scale and bias, in float64.

Test infrastructure: part of the CPU oracle (see the package docstring for who
may import it).

The steps follow the HunyuanVideo1.5 retrospective (aigcage.com, section 3.1): the
bf16 activation is quantised to FP8 with one scale per token, multiplied with the
FP8 weight, and the product is scaled, biased and converted to the output type. The
weight is nn.Linear's [N, K] with K contiguous (the column-major B operand of that
section), so the product is C = A @ W^T.

Exactness of the float64 product: every e4m3fn value is an integer multiple of
2^-9 with magnitude <= 448, so each product is a multiple of 2^-18 below 2^18 in
magnitude. For K <= 2^17 every partial sum is an integer below 2^53 in units of
2^-18, so float64 holds the exact dot product in any summation order (a BLAS
matmul included). The oracle's reference output is left unrounded in float64;
tests compare the GPU's bf16 output against it.

A row of A may also arrive already quantised with its scale (section 3.5 of the
same page: an input that is already float8_e4m3fn is used with the scale passed
in); ``linear_ref_fp8`` is that entry.
"""

import numpy as np

from . import e4m3, quant

MAX_EXACT_K = 1 << 17


def gemm_exact(qa, qw):
    """acc[m, n] = sum_k dec(qa[m, k]) * dec(qw[n, k]), exact, float64 [M, N]."""
    qa = np.asarray(qa, dtype=np.uint8)
    qw = np.asarray(qw, dtype=np.uint8)
    if qa.ndim != 2 or qw.ndim != 2 or qa.shape[1] != qw.shape[1]:
        raise ValueError("gemm_exact expects qa [M, K] and qw [N, K]")
    if qa.shape[1] > MAX_EXACT_K:
        raise ValueError("float64 exactness argument holds for K <= 2^17")
    return e4m3.decode(qa) @ e4m3.decode(qw).T


def epilogue(acc, a_scale, w_scale, bias_bits=None):
    """out[m, n] = acc[m, n] * a_scale[m] * w_scale[n] + bias[n], float64, unrounded."""
    out = np.asarray(acc, dtype=np.float64) * np.asarray(a_scale, dtype=np.float32).astype(np.float64)[:, None]
    out = out * np.asarray(w_scale, dtype=np.float32).astype(np.float64)[None, :]
    if bias_bits is not None:
        out = out + quant.bf16_bits_to_f32(bias_bits).astype(np.float64)[None, :]
    return out


def linear_ref_fp8(qa, a_scale, qw, w_scale, bias_bits=None):
    """Linear on an activation that is already (e4m3fn codes, per-row scale)."""
    return epilogue(gemm_exact(qa, qw), a_scale, w_scale, bias_bits)


def linear_ref(a_bits, qw, w_scale, bias_bits=None):
    """Linear on a bf16 activation (uint16 bits [M, K]): per-token quant, FP8 product, epilogue.

    Returns (out float64 [M, N], qa uint8 [M, K], a_scale float32 [M]).
    """
    qa, sa = quant.quant_rows(a_bits)
    return linear_ref_fp8(qa, sa, qw, w_scale, bias_bits), qa, sa
