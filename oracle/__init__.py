"""float64 CPU oracle for single-precision GEMM (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never imports, links or
calls it, and it imports nothing from the HIP library: the two share no code.

What it computes is the plain definition of GEMM,

    C_out[i][j] = alpha * sum_k A[i][k] * B[k][j] + beta * C_in[i][j],

for row-major fp32 A (M x K), B (K x N), C (M x N) with leading dimensions
lda, ldb, ldc ("SGEMM CUDA kernel (First Half)", introduction and "Part 1: CPU
version"; "Optimizing Matrix Multiplication in CUDA", "Baseline CPU
Implementation").  Every function returns ``(ref, bound)`` in float64, where a
GPU value g passes when ``|g - ref| <= bound`` with

    bound = 1e-5 * (|alpha| * sum_k |a_ik * b_kj| + |beta * c_ij|) + 1e-6.

Two forms are provided:

* ``ref_rows`` / ``ref_points`` -- the i-j-k triple loop in C (``sgemm_ref.c``),
  float64 accumulation in ascending k, OpenMP over rows.  This is the oracle.
* ``ref_matmul`` -- the same definition with numpy's float64 matrix product as
  the one library step, for full-size checks where the triple loop is too slow.
  Its rounding order differs from the loop's (still ~1e-16 relative, far inside
  the bound) and it is exact on integer-valued inputs.

Conventions (readings of the pages, see sgemm_ref.c): beta == 0 never reads C;
alpha == 0 or K == 0 never reads A or B and gives beta * C.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sgemm_ref.c")
_LIB = os.path.join(_HERE, "libsgemm_ref.so")
_lock = threading.Lock()
_lib = None

REL_TOL = 1e-5
ABS_TOL = 1e-6


def build(verbose: bool = False) -> str:
    """Compile sgemm_ref.c into libsgemm_ref.so (gcc, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           _SRC, "-o", _LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        f = ctypes.c_void_p
        i = ctypes.c_int
        lng = ctypes.c_long
        d = ctypes.c_double
        lib.sgemm_ref_rows.argtypes = [i, i, i, d, f, lng, f, lng, d, f, lng, i, i, f, f, i]
        lib.sgemm_ref_rows.restype = i
        lib.sgemm_ref_points.argtypes = [i, i, i, d, f, lng, f, lng, d, f, lng, f, f, lng, f, f, i]
        lib.sgemm_ref_points.restype = i
        lib.sgemm_ref_max_threads.argtypes = []
        lib.sgemm_ref_max_threads.restype = i
        _lib = lib
        return lib


def max_threads() -> int:
    """Threads an OpenMP region of the oracle uses by default."""
    return int(_load().sgemm_ref_max_threads())


def _mat(x, name):
    """Return (pointer, ld, rows, cols) of a 2-D float32 row-major array (possibly a padded view)."""
    if x is None:
        return None, 1, 0, 0
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.size == 0:  # an empty operand is never read
        return ctypes.c_void_p(x.ctypes.data), max(1, x.shape[1]), x.shape[0], x.shape[1]
    if x.shape[1] > 1 and x.strides[1] != 4:
        raise ValueError(f"{name} must have unit column stride")
    ld = x.strides[0] // 4 if x.shape[0] > 1 else max(1, x.shape[1])
    if x.strides[0] % 4 != 0 or ld < max(1, x.shape[1]):
        raise ValueError(f"{name} has an invalid row stride")
    return ctypes.c_void_p(x.ctypes.data), ld, x.shape[0], x.shape[1]


def _shapes(A, B, C, alpha, beta, M=None, N=None, K=None):
    pa, lda, ma, ka = _mat(A, "A")
    pb, ldb, kb, nb = _mat(B, "B")
    pc, ldc, mc, nc = _mat(C, "C")
    M = M if M is not None else (ma if A is not None else mc)
    N = N if N is not None else (nb if B is not None else nc)
    K = K if K is not None else (ka if A is not None else kb)
    if A is not None and (ma, ka) != (M, K):
        raise ValueError("A shape mismatch")
    if B is not None and (kb, nb) != (K, N):
        raise ValueError("B shape mismatch")
    if C is not None and (mc, nc) != (M, N):
        raise ValueError("C shape mismatch")
    if beta != 0.0 and C is None and M * N > 0:
        raise ValueError("C is required when beta != 0")
    if alpha != 0.0 and K > 0 and M * N > 0 and (A is None or B is None):
        raise ValueError("A and B are required when alpha != 0 and K > 0")
    return M, N, K, pa, lda, pb, ldb, pc, ldc


def ref_rows(A, B, C, alpha=1.0, beta=0.0, rows=None, nthreads=0, M=None, N=None, K=None):
    """Reference rows [r0, r1) of C_out (all rows by default) -> (ref, bound), each (r1-r0) x N float64."""
    M, N, K, pa, lda, pb, ldb, pc, ldc = _shapes(A, B, C, alpha, beta, M, N, K)
    r0, r1 = (0, M) if rows is None else rows
    ref = np.empty((r1 - r0, N), dtype=np.float64)
    bound = np.empty((r1 - r0, N), dtype=np.float64)
    rc = _load().sgemm_ref_rows(M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc,
                                r0, r1, ctypes.c_void_p(ref.ctypes.data),
                                ctypes.c_void_p(bound.ctypes.data), int(nthreads))
    if rc != 0:
        raise ValueError(f"sgemm_ref_rows rejected its arguments ({rc})")
    return ref, bound


def ref_points(A, B, C, I, J, alpha=1.0, beta=0.0, nthreads=0, M=None, N=None, K=None):
    """Reference at the elements (I[p], J[p]) -> (ref, bound), each of length len(I)."""
    M, N, K, pa, lda, pb, ldb, pc, ldc = _shapes(A, B, C, alpha, beta, M, N, K)
    I = np.ascontiguousarray(I, dtype=np.int64)
    J = np.ascontiguousarray(J, dtype=np.int64)
    if I.shape != J.shape or I.ndim != 1:
        raise ValueError("I and J must be 1-D of equal length")
    ref = np.empty(I.shape[0], dtype=np.float64)
    bound = np.empty(I.shape[0], dtype=np.float64)
    rc = _load().sgemm_ref_points(M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc,
                                  ctypes.c_void_p(I.ctypes.data), ctypes.c_void_p(J.ctypes.data),
                                  I.shape[0], ctypes.c_void_p(ref.ctypes.data),
                                  ctypes.c_void_p(bound.ctypes.data), int(nthreads))
    if rc != 0:
        raise ValueError(f"sgemm_ref_points rejected its arguments ({rc})")
    return ref, bound


def ref_matmul(A, B, C, alpha=1.0, beta=0.0):
    """Full reference via numpy float64 matrix products -> (ref, bound), each M x N float64.

    Same definition and conventions as the triple loop; the sums come from a
    library float64 matmul (A64 @ B64, and |A64| @ |B64| for the bound).
    """
    A = None if A is None else np.asarray(A)
    B = None if B is None else np.asarray(B)
    C = None if C is None else np.asarray(C)
    M = A.shape[0] if A is not None else C.shape[0]
    N = B.shape[1] if B is not None else C.shape[1]
    K = A.shape[1] if A is not None else (B.shape[0] if B is not None else 0)
    if alpha != 0.0 and K > 0:
        A64 = A.astype(np.float64)
        B64 = B.astype(np.float64)
        s = A64 @ B64
        sa = np.abs(A64) @ np.abs(B64)
        del A64, B64
    else:
        s = np.zeros((M, N), dtype=np.float64)
        sa = np.zeros((M, N), dtype=np.float64)
    c = beta * C.astype(np.float64) if beta != 0.0 else np.zeros((M, N), dtype=np.float64)
    ref = alpha * s + c
    bound = REL_TOL * (abs(alpha) * sa + np.abs(c)) + ABS_TOL
    return ref, bound
