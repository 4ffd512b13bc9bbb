"""Cache-blocked, multi-threaded CPU SGEMM: a second CPU baseline for bench.py.

The plain float64 oracle (``oracle/``) is the correctness reference and a deliberately
naive CPU figure; this is the fair CPU figure next to it: fp32, packed panels, an MR x NR
register tile with AVX-512 or AVX2 fused multiply-adds (chosen at run time), OpenMP over
row blocks.  Measurement only: the GPU library never calls it, and tests check it against
the oracle (it is never the expected value of anything).

    C := alpha * A @ B + beta * C      (row-major fp32, leading dimensions)

Why: "Shared Memory and Register Blocking" (CUDA Handbook, ch. 17) sets a cache-blocked CPU
product against a plain loop to show how much the plain loop understates the CPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgemm_blocked.c")
_LIB = os.path.join(_HERE, "libsgemm_blocked.so")
_lock = threading.Lock()
_lib = None


def build(verbose: bool = False) -> str:
    """Compile sgemm_blocked.c (gcc -O3, OpenMP; the SIMD tile is chosen at run time)."""
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           _SRC, "-o", _LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
            i, f, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
            lib.sgemm_blocked.argtypes = [i, i, i, f, vp, i, vp, i, f, vp, i, i]
            lib.sgemm_blocked.restype = i
            lib.sgemm_blocked_isa.argtypes = []
            lib.sgemm_blocked_isa.restype = i
            _lib = lib
        return _lib


def isa() -> str:
    """The SIMD form of the register tile on this CPU."""
    return {2: "avx512", 1: "avx2+fma", 0: "portable C"}[_load().sgemm_blocked_isa()]


def _mat(x: np.ndarray, name: str):
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.size == 0:
        return None, max(1, x.shape[1])
    if x.shape[1] > 1 and x.strides[1] != 4:
        raise ValueError(f"{name} must have unit column stride")
    ld = x.strides[0] // 4 if x.shape[0] > 1 else max(1, x.shape[1])
    return x.ctypes.data, max(ld, x.shape[1], 1)


def gemm(A: np.ndarray, B: np.ndarray, C: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
         nthreads: int = 0) -> np.ndarray:
    """C := alpha*A@B + beta*C in place (C must be writeable); returns C."""
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or C.shape != (M, N):
        raise ValueError("shape mismatch")
    if not C.flags.writeable:
        raise ValueError("C must be writeable")
    pa, lda = _mat(A, "A")
    pb, ldb = _mat(B, "B")
    pc, ldc = _mat(C, "C")
    rc = _load().sgemm_blocked(M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"sgemm_blocked returned {rc}")
    return C
