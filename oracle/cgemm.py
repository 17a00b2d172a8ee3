"""Builder and ctypes loader for ``oracle_gemm.c`` (test infrastructure only).

``build()`` compiles the C source with gcc (OpenMP) into
``oracle/liboracle_gemm.so``; ``gemm()`` calls it on numpy int64 limb arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB = os.path.join(_HERE, "liboracle_gemm.so")
_lib = None


def build() -> str:
    """Compile the C oracle (always recompiles).  Returns the library path."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, _SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemm.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def gemm(A: np.ndarray, B: np.ndarray, lc: int) -> np.ndarray:
    """Exact C = A @ B.  A: int64 [M,K,la], B: int64 [K,N,lb] -> int64 [M,N,lc].

    Raises OverflowError if some entry does not fit ``lc`` limbs.
    """
    A = np.ascontiguousarray(A, dtype=np.int64)
    B = np.ascontiguousarray(B, dtype=np.int64)
    assert A.ndim == 3 and B.ndim == 3 and A.shape[1] == B.shape[0]
    M, K, la = A.shape
    _, N, lb = B.shape
    C = np.zeros((M, N, lc), dtype=np.int64)
    rc = _load().oracle_gemm(M, N, K, A.ctypes.data, la, B.ctypes.data, lb, C.ctypes.data, lc)
    if rc == 1:
        raise OverflowError("result does not fit the requested limbs")
    if rc != 0:
        raise ValueError(f"oracle_gemm failed with code {rc}")
    return C


def threads_used() -> int:
    """OpenMP threads the C oracle runs with (OMP_NUM_THREADS, else affinity)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))
