"""ctypes access to oracle/csrc/quant_ref.c, the C statement of the per-row quantisation.

Test infrastructure: part of the CPU oracle (only tests/, smoke() and the bench's
cpu_baseline may use it). It exists for sweeps too large for numpy (the
exhaustive bf16 (x, amax) sweep); tests pin it bit-for-bit to oracle.quant.
``build()`` compiles it with gcc; nothing here is shared with the HIP library.
"""

import ctypes
import os
import shutil
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "quant_ref.c")
LIB = os.path.join(HERE, "liboracle_quant_ref.so")

_lib = None


def build():
    """Compile the C oracle with plain IEEE arithmetic (no fast-math, no contraction)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C oracle")
    tmp = LIB + ".tmp"
    subprocess.run([cc, "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", SRC,
                    "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        h = ctypes.CDLL(LIB)
        h.oracle_quant_rows_bf16.restype = None
        h.oracle_quant_rows_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_void_p]
        h.oracle_encode_e4m3fn.restype = ctypes.c_uint8
        h.oracle_encode_e4m3fn.argtypes = [ctypes.c_float]
        _lib = h
    return _lib


def quant_rows(x_bits):
    """Same contract as oracle.quant.quant_rows (uint16 bf16 bits [R, C] -> codes, scales)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows,), np.float32)
    lib().oracle_quant_rows_bf16(x.ctypes.data, rows, cols, q.ctypes.data, s.ctypes.data)
    return q, s
