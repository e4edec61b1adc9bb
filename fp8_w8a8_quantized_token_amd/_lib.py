"""ctypes loader for libfp8w8a8.so: symbol declarations and status handling.

The library is the only implementation: if it is missing or fails to load, the
import of any op raises; nothing here computes anything itself.
"""

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfp8w8a8.so")

# status codes (include/fp8w8a8.h)
OK = 0
ERR_INVALID_ARG = -1
ERR_BAD_SHAPE = -2
ERR_MISALIGNED = -3
ERR_BAD_DEVICE = -4
ERR_WORKSPACE_TOO_SMALL = -5
ERR_HIP = -6
ERR_CAPTURE = -7
ERR_TOO_LARGE = -8

A_BF16 = 0
A_E4M3 = 1

ACT_GELU_ERF = 1
ACT_GELU_TANH = 2
ACT_SILU = 3
ACT_TABLE_BYTES = 131072

FMT_E4M3FN = 0
FMT_E5M2 = 1

TENSOR_FORMS = {"auto": 0, "one_pass": 1, "two_pass": 2, "one_pass_no_wait": 3}

NOALLOC_SCRATCH_BYTES = 80 << 20

MAX_ROWS = 1 << 24
MAX_GROUP = 4
MAX_DIM = 1 << 20

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p

# name -> (restype, argtypes); every function declared in include/fp8w8a8.h
SIGNATURES = {
    "fp8w8a8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp8_quant_rows": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "fp8_quant_weights_per_channel": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "fp8_act_table_build": (ctypes.c_int, [ctypes.c_int, _c_p, _c_p]),
    "fp8_quant_tensor_workspace_bytes": (ctypes.c_size_t, []),
    "fp8_quant_tensor": (ctypes.c_int, [_c_p, _c_i64, ctypes.c_int, _c_p, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "fp8_quant_tensor_form": (ctypes.c_int, [ctypes.c_int, _c_p, _c_i64, ctypes.c_int, _c_p, _c_p, _c_p,
                                             ctypes.c_size_t, _c_p]),
    "fp8_dequant_tensor": (ctypes.c_int, [_c_p, _c_i64, ctypes.c_int, _c_p, _c_p, _c_p]),
    "fp8_act_rows": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "fp8_act_quant_rows": (ctypes.c_int, [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "fp8_linear_create": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_p, _c_p, _c_p, ctypes.POINTER(_c_p)]),
    "fp8_linear_workspace_bytes": (ctypes.c_size_t, [_c_p, _c_i64]),
    "fp8_linear_run": (ctypes.c_int, [_c_p, _c_i64, _c_p, ctypes.c_int, _c_p, _c_p, _c_p, ctypes.c_size_t, _c_p]),
    "fp8_linear_run_noalloc": (ctypes.c_int, [_c_p, _c_i64, _c_p, ctypes.c_int, _c_p, _c_p, _c_p]),
    "fp8_linear_run_group": (ctypes.c_int, [_c_p, ctypes.c_int, _c_i64, _c_p, ctypes.c_int, _c_p, _c_p, _c_p,
                                            ctypes.c_size_t, _c_p]),
    "fp8_linear_destroy": (None, [_c_p]),
    "fp8_linear": (ctypes.c_int, [_c_p, ctypes.c_int, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p,
                                  ctypes.c_size_t, _c_p]),
    "fp8_linear_plan_config": (ctypes.c_int, [_c_p, _c_i64, ctypes.POINTER(ctypes.c_int),
                                              ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                              ctypes.POINTER(_c_i64)]),
    "fp8_linear_group_config": (ctypes.c_int, [_c_p, ctypes.c_int, _c_i64, ctypes.POINTER(ctypes.c_int)]),
    "fp8_gemm_config_count": (ctypes.c_int, []),
    "fp8_w8a16_create": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, ctypes.c_int, _c_p, _c_p, _c_p,
                                         ctypes.POINTER(_c_p)]),
    "fp8_w8a16_run": (ctypes.c_int, [_c_p, _c_i64, _c_p, _c_p, _c_p]),
    "fp8_w8a16_destroy": (None, [_c_p]),
    "fp8_w8a16_plan_config": (ctypes.c_int, [_c_p, _c_i64, ctypes.POINTER(ctypes.c_int),
                                             ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                             ctypes.POINTER(_c_i64)]),
    "fp8_w8a16_config_count": (ctypes.c_int, []),
    "fp8_w8a16_run_config": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p,
                                            _c_p, _c_p, _c_p]),
    "fp8_gemm_run_config": (ctypes.c_int, [ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p,
                                           _c_p, _c_p]),
    "fp8_quant_gemm_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "fp8_quant_gemm": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_size_t,
                                      _c_p]),
}


class Fp8W8A8Error(RuntimeError):
    """A non-zero status from libfp8w8a8."""

    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib():
    """Load libfp8w8a8.so once and declare its symbols; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m fp8_w8a8_quantized_token_amd.build` "
                "(there is no other implementation to fall back to)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status):
    return lib().fp8w8a8_status_string(int(status)).decode()


def check(status, where):
    if status != OK:
        raise Fp8W8A8Error(status, where)
