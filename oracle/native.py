"""Builds and loads the C parts of the oracle (plain gcc, no GPU code).

TEST INFRASTRUCTURE ONLY (see the package header)."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c", "nvfp4_search.c")
LIB = os.path.join(HERE, "c", "liboracle_nvfp4.so")
_lib = None


def build() -> str:
    """Compile the C oracle (IEEE float64, no contraction, OpenMP over blocks)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           SRC, "-o", LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        l = ctypes.CDLL(LIB)
        l.nvfp4_choose_scales.restype = None
        l.nvfp4_choose_scales.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
        l.nvfp4_block_error.restype = ctypes.c_double
        l.nvfp4_block_error.argtypes = [ctypes.c_void_p, ctypes.c_double]
        _lib = l
    return _lib
