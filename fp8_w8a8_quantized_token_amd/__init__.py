"""MI355X-native FP8 W8A8 linear layer: per-token e4m3fn activation quantisation,
FP8 MFMA GEMM against per-channel e4m3fn weights, fused scale/bias/bf16 epilogue.

The compute lives in libfp8w8a8.so (HIP kernels for gfx950 behind a C ABI, see
include/fp8w8a8.h); this package is the thin torch binding around it. Build the
library with ``python -m fp8_w8a8_quantized_token_amd.build``.
"""

from ._lib import Fp8W8A8Error, LIB_PATH, lib  # noqa: F401
from .ops import (  # noqa: F401
    A_BF16,
    A_E4M3,
    ACTIVATIONS,
    Fp8Linear,
    Fp8WeightOnlyLinear,
    act_quant_rows,
    act_rows,
    act_table,
    dequant_tensor,
    quant_tensor,
    gemm_config_count,
    gemm_run_config,
    linear,
    group_config,
    linear_group,
    quant_gemm,
    quant_rows,
    quant_weights_per_channel,
    w8a16_config_count,
    w8a16_run_config,
)

__all__ = [
    "Fp8Linear",
    "Fp8W8A8Error",
    "Fp8WeightOnlyLinear",
    "w8a16_config_count",
    "w8a16_run_config",
    "ACTIVATIONS",
    "act_table",
    "act_rows",
    "act_quant_rows",
    "quant_tensor",
    "dequant_tensor",
    "linear",
    "group_config",
    "linear_group",
    "quant_rows",
    "quant_weights_per_channel",
    "gemm_config_count",
    "gemm_run_config",
    "quant_gemm",
    "lib",
    "LIB_PATH",
    "A_BF16",
    "A_E4M3",
]
