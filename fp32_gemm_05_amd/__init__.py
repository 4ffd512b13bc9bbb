"""libsgemm: single-precision GEMM (C = alpha*op(A)*op(B) + beta*C, row-major fp32) for MI355X.

The compute path is hand-written HIP for gfx950 behind a C ABI
(``include/sgemm.h``, ``libsgemm.so``); this package is the thin ctypes binding
over it.  Importing the package loads nothing: the shared library is opened on
the first call, and a missing library raises instead of falling back to any
other implementation.
"""
from ._binding import (  # noqa: F401
    SgemmArgumentError,
    SgemmError,
    SgemmLaunchError,
    gemm,
    library_path,
    load_library,
    sgemm,
    sgemm_ex,
    sgemm_last_variant,
    sgemm_num_variants,
    sgemm_op,
    sgemm_op_ex,
    sgemm_op_select_variant,
    sgemm_select_variant,
    sgemm_variant_info,
    sgemm_variant_name,
    sgemm_version,
    tile_order,
)
