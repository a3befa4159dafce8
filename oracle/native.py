"""ctypes loader for the plain-C part of the oracle (test infrastructure only).

`build()` compiles oracle/c/*.c with gcc into oracle/_oracle_c.so; `load()`
compiles only when no library is present.
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "c", "nearest_level.c")
_LIB = os.path.join(_HERE, "_oracle_c.so")
_handle = None


def build() -> str:
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def load():
    global _handle
    if _handle is not None:
        return _handle
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_nearest_level.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p]
    lib.oracle_nearest_level.restype = None
    lib.oracle_nearest_level_bits.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p,
                                              ctypes.c_int, ctypes.c_void_p]
    lib.oracle_nearest_level_bits.restype = None
    _handle = lib
    return lib


def nearest_level(x: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Same definition as oracle.nf4.nearest_level, in C."""
    lib = load()
    xs = np.ascontiguousarray(x, dtype=np.float32)
    lv = np.ascontiguousarray(levels, dtype=np.float32)
    out = np.empty(xs.shape, dtype=np.uint8)
    lib.oracle_nearest_level(xs.ctypes.data, xs.size, lv.ctypes.data, lv.size, out.ctypes.data)
    return out


def nearest_level_of_bits(first_bits: int, n: int, levels: np.ndarray) -> np.ndarray:
    """Codes of the n consecutive fp32 bit patterns starting at first_bits."""
    lib = load()
    lv = np.ascontiguousarray(levels, dtype=np.float32)
    out = np.empty(n, dtype=np.uint8)
    lib.oracle_nearest_level_bits(first_bits, n, lv.ctypes.data, lv.size, out.ctypes.data)
    return out
