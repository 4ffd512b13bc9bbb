"""ctypes binding of libsgemm's C ABI (argument marshalling only).

Every function mirrors the C entry point of the same name in include/sgemm.h.
Matrices may be passed as device addresses (int) or as torch CUDA tensors,
whose ``data_ptr()`` is used.  ``stream=None`` means torch's current stream on
the current device.  No arithmetic happens here: a missing or unloadable
library raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsgemm.so")
_lock = threading.Lock()
_lib = None

_ARG_NAMES = {1: "M", 2: "N", 3: "K", 4: "alpha", 5: "A", 6: "lda", 7: "B", 8: "ldb", 9: "beta",
              10: "C", 11: "ldc", 12: "stream", 13: "variant"}
# sgemm_op / sgemm_op_ex number the two transposition characters first
_OP_ARG_NAMES = {1: "transa", 2: "transb", **{k + 2: v for k, v in _ARG_NAMES.items()}}


class SgemmError(RuntimeError):
    """A non-zero return code of the C ABI (``code`` holds it).  Raised as one of the two
    subclasses below."""

    def __init__(self, code: int, where: str):
        self.code = code
        if code < 0:
            names = _OP_ARG_NAMES if where.startswith("sgemm_op") else _ARG_NAMES
            what = f"argument {-code} ({names.get(-code, '?')}) is invalid"
        else:
            what = f"kernel launch failed with hipError_t {code}"
        super().__init__(f"{where}: {what}")


class SgemmArgumentError(SgemmError, ValueError):
    """A negative return code: argument ``-code`` is invalid; nothing was enqueued."""


class SgemmLaunchError(SgemmError):
    """A positive return code: the kernel launch failed with that hipError_t."""


def _error(code: int, where: str) -> SgemmError:
    return (SgemmArgumentError if code < 0 else SgemmLaunchError)(code, where)


def library_path() -> str:
    return _LIB_PATH


def load_library(path: str | None = None):
    """Open libsgemm.so (built in-tree by ``fp32_gemm_05_amd.build``); raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or _LIB_PATH
        if not os.path.exists(p):
            raise FileNotFoundError(
                f"{p} is not built; run `python -m fp32_gemm_05_amd.build` or __graft_entry__.build()")
        lib = ctypes.CDLL(p)
        i, f, vp, cp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_char_p
        gemm_args = [i, i, i, f, vp, i, vp, i, f, vp, i, vp]
        lib.sgemm.argtypes = gemm_args
        lib.sgemm.restype = i
        lib.sgemm_ex.argtypes = gemm_args + [i]
        lib.sgemm_ex.restype = i
        ch = ctypes.c_char
        lib.sgemm_op.argtypes = [ch, ch] + gemm_args
        lib.sgemm_op.restype = i
        lib.sgemm_op_ex.argtypes = [ch, ch] + gemm_args + [i]
        lib.sgemm_op_ex.restype = i
        lib.sgemm_op_select_variant.argtypes = [ch, ch, i, i, i, vp, i, vp, i, vp, i]
        lib.sgemm_op_select_variant.restype = i
        lib.sgemm_num_variants.argtypes = []
        lib.sgemm_num_variants.restype = i
        lib.sgemm_variant_name.argtypes = [i]
        lib.sgemm_variant_name.restype = cp
        lib.sgemm_variant_info.argtypes = [i, ctypes.POINTER(i), i]
        lib.sgemm_variant_info.restype = i
        lib.sgemm_select_variant.argtypes = [i, i, i, vp, i, vp, i, vp, i]
        lib.sgemm_select_variant.restype = i
        lib.sgemm_tile_order.argtypes = [i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
        lib.sgemm_tile_order.restype = i
        lib.sgemm_last_variant.argtypes = []
        lib.sgemm_last_variant.restype = i
        lib.sgemm_version.argtypes = []
        lib.sgemm_version.restype = cp
        if path is None:
            _lib = lib
        return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"expected a device address or a tensor, got {type(x).__name__}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # a torch.cuda.Stream


def sgemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """C := alpha*A*B + beta*C on the device (see include/sgemm.h). Raises SgemmError on a non-zero code."""
    rc = load_library().sgemm(int(M), int(N), int(K), float(alpha), _ptr(A), int(lda), _ptr(B), int(ldb),
                              float(beta), _ptr(C), int(ldc), _stream(stream))
    if rc != 0:
        raise _error(rc, "sgemm")


def sgemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None, variant=-1):
    """sgemm with a forced kernel variant (variant < 0: choose as sgemm does)."""
    rc = load_library().sgemm_ex(int(M), int(N), int(K), float(alpha), _ptr(A), int(lda), _ptr(B), int(ldb),
                                 float(beta), _ptr(C), int(ldc), _stream(stream), int(variant))
    if rc != 0:
        raise _error(rc, "sgemm_ex")


def _trans(t) -> bytes:
    if isinstance(t, bool):
        return b"T" if t else b"N"
    if isinstance(t, str) and len(t) == 1:
        return t.encode()
    if isinstance(t, bytes) and len(t) == 1:
        return t
    raise TypeError(f"transposition must be one character or a bool, got {t!r}")


def sgemm_op(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """C := alpha*op(A)*op(B) + beta*C; transa/transb 'N' or 'T' (or bools). Raises SgemmError."""
    rc = load_library().sgemm_op(_trans(transa), _trans(transb), int(M), int(N), int(K), float(alpha), _ptr(A),
                                 int(lda), _ptr(B), int(ldb), float(beta), _ptr(C), int(ldc), _stream(stream))
    if rc != 0:
        raise _error(rc, "sgemm_op")


def sgemm_op_ex(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None, variant=-1):
    """sgemm_op with a forced kernel variant (variant < 0: choose as sgemm_op does)."""
    rc = load_library().sgemm_op_ex(_trans(transa), _trans(transb), int(M), int(N), int(K), float(alpha),
                                    _ptr(A), int(lda), _ptr(B), int(ldb), float(beta), _ptr(C), int(ldc),
                                    _stream(stream), int(variant))
    if rc != 0:
        raise _error(rc, "sgemm_op_ex")


def sgemm_num_variants() -> int:
    return int(load_library().sgemm_num_variants())


def sgemm_variant_name(variant: int):
    s = load_library().sgemm_variant_name(int(variant))
    return None if s is None else s.decode()


def sgemm_variant_info(variant: int) -> dict:
    info = (ctypes.c_int * 17)()
    if load_library().sgemm_variant_info(int(variant), info, 17) != 0:
        raise ValueError(f"no variant {variant}")
    keys = ["kind", "BM", "BN", "BK", "WM_or_TM", "WN_or_TN", "threads", "vec", "lds_bytes", "wide", "ksplit",
            "trans_a", "trans_b", "b_kquad", "dl_stages", "persistent", "mfma_block"]
    d = dict(zip(keys, list(info)))
    d["kind"] = "mfma" if d["kind"] == 0 else "valu"
    d["name"] = sgemm_variant_name(variant)
    return d


def sgemm_select_variant(M, N, K, A, lda, B, ldb, C, ldc) -> int:
    return int(load_library().sgemm_select_variant(int(M), int(N), int(K), _ptr(A), int(lda), _ptr(B),
                                                   int(ldb), _ptr(C), int(ldc)))


def sgemm_op_select_variant(transa, transb, M, N, K, A, lda, B, ldb, C, ldc) -> int:
    return int(load_library().sgemm_op_select_variant(_trans(transa), _trans(transb), int(M), int(N), int(K),
                                                      _ptr(A), int(lda), _ptr(B), int(ldb), _ptr(C), int(ldc)))


def sgemm_last_variant() -> int:
    """Variant id of this thread's most recent computing call, or -1 (see include/sgemm.h)."""
    return int(load_library().sgemm_last_variant())


def sgemm_version() -> str:
    return load_library().sgemm_version().decode()


def tile_order(tiles_m: int, tiles_n: int, group_m: int):
    """Host copy of the kernels' workgroup -> tile map: lists (tile_m, tile_n) indexed by workgroup id."""
    n = tiles_m * tiles_n
    tm = (ctypes.c_int * n)()
    tn = (ctypes.c_int * n)()
    if load_library().sgemm_tile_order(int(tiles_m), int(tiles_n), int(group_m), tm, tn) != 0:
        raise ValueError("bad tile grid")
    return list(tm), list(tn)


def _require_device(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _check_matrix(t, name):
    """Validate a 2-D float32 device tensor with unit column stride; returns its leading dimension."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != torch.float32 or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float32 tensor")
    _require_device(t, name)
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must be row-major with unit column stride")
    if t.shape[0] <= 1 or t.shape[1] == 0:
        return max(1, t.shape[1])  # one row, or no element: no stride is addressed
    if t.stride(0) < t.shape[1]:
        # a broadcast (stride 0) or overlapping view: its rows share storage, so no leading
        # dimension describes it, and the library would address past its storage
        raise ValueError(f"{name} has row stride {t.stride(0)} below its row length {t.shape[1]} "
                         f"(a broadcast or overlapping view); pass a contiguous copy")
    return t.stride(0)


def _column_major(t) -> bool:
    """A 2-D view with unit row stride (e.g. ``x.t()`` of a row-major x): its transpose is row-major."""
    return t.dim() == 2 and t.shape[0] > 1 and t.shape[1] > 1 and t.stride(0) == 1 and t.stride(1) >= t.shape[0]


def gemm(A, B, C, alpha: float = 1.0, beta: float = 0.0, variant: int = -1, stream=None,
         trans_a: bool = False, trans_b: bool = False):
    """Tensor form: C := alpha*op(A)@op(B) + beta*C in place for 2-D float32 device tensors; returns C.

    A and B are the stored row-major arrays; ``trans_a`` reads A (K x M) as A^T, ``trans_b`` reads
    B (N x K) as B^T.  Column-major views (unit row stride, such as ``x.t()``) are accepted without
    a copy: an operand view is passed as its row-major storage with the transposition flipped, and
    a column-major C is computed as C^T := alpha*op(B)^T@op(A)^T + beta*C^T on its storage (with
    ``variant`` < 0 only, since the roles of A and B swap)."""
    if _column_major(C):
        if variant >= 0:
            raise ValueError("a forced variant needs a row-major C")
        # C^T = op(B)^T op(A)^T: B takes A's place with the opposite flag, and A takes B's
        gemm(B, A, C.t(), alpha, beta, -1, stream, trans_a=not trans_b, trans_b=not trans_a)
        return C
    if _column_major(A):
        A, trans_a = A.t(), not trans_a
    if _column_major(B):
        B, trans_b = B.t(), not trans_b
    lda = _check_matrix(A, "A")
    ldb = _check_matrix(B, "B")
    ldc = _check_matrix(C, "C")
    M, K = (A.shape[1], A.shape[0]) if trans_a else tuple(A.shape)
    K2, N = (B.shape[1], B.shape[0]) if trans_b else tuple(B.shape)
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    if trans_a or trans_b:
        sgemm_op_ex(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant)
    else:
        sgemm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant)
    return C
