"""Helpers shared by the GPU tests: device buffers with padding/sentinels and oracle comparisons."""
from __future__ import annotations

import numpy as np

SENTINEL = 12345.0  # finite marker around C: any stray write changes it


def device_matrix(x: np.ndarray, pad_cols: int = 0, pad_rows: int = 0, offset: int = 0,
                  fill: float = float("nan"), device="cuda"):
    """Copy x into a device buffer of row stride cols+pad_cols, starting `offset` floats in.

    Returns (buf, view, ld): `buf` is the whole 1-D allocation (filled with
    `fill` outside x), `view` the (rows, cols) strided view holding x.
    """
    import torch
    rows, cols = x.shape
    ld = max(1, cols + pad_cols)
    n = offset + (rows + pad_rows) * ld
    buf = torch.full((max(n, 1),), fill, dtype=torch.float32, device=device)
    view = buf[offset:offset + rows * ld].view(rows, ld)[:, :cols]
    if x.size:
        view.copy_(torch.from_numpy(np.ascontiguousarray(x)))
    return buf, view, ld


def outside_mask(rows: int, cols: int, ld: int, pad_rows: int, offset: int, n: int):
    """Boolean mask over a 1-D buffer of length n: True where the element is NOT part of the matrix."""
    m = np.ones(n, dtype=bool)
    for r in range(rows):
        m[offset + r * ld: offset + r * ld + cols] = False
    return m


def check_within_bound(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str = "") -> float:
    """Assert |got - ref| <= bound element-wise and everything is finite; returns max err/bound."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    finite = np.isfinite(got)
    assert finite.all(), f"{what}: {np.count_nonzero(~finite)} non-finite outputs, first at " \
                         f"{np.argwhere(~finite)[:3].tolist()}"
    err = np.abs(got - ref)
    ratio = err / bound
    worst = float(ratio.max())
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        bad = np.count_nonzero(ratio > 1.0)
        raise AssertionError(f"{what}: {bad} elements outside the bound; worst at {idx}: got {got[idx]!r}, "
                             f"ref {ref[idx]!r}, bound {bound[idx]!r} (err/bound {worst:.3g})")
    return worst


def check_exact(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """Assert got == ref by value (so +0 == -0), for integer-valued results."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    neq = got != ref
    if neq.any():
        idx = tuple(np.argwhere(neq)[0])
        raise AssertionError(f"{what}: {np.count_nonzero(neq)} elements differ; first at {idx}: "
                             f"got {got[idx]!r}, want {ref[idx]!r}")


def assert_border_untouched(buf_host: np.ndarray, rows: int, cols: int, ld: int, offset: int = 0,
                            sentinel: float = SENTINEL, what: str = ""):
    """Every element of a 1-D host copy of C's buffer outside the rows x cols window (row stride
    ld, starting `offset` floats in) still holds the sentinel.  Vectorised: full-size C has up to
    hundreds of thousands of rows."""
    inside = np.zeros(buf_host.shape[0], dtype=bool)
    if rows and cols:
        starts = offset + np.arange(rows, dtype=np.int64) * ld
        idx = (starts[:, None] + np.arange(cols, dtype=np.int64)[None, :]).ravel()
        inside[idx] = True
    outside = buf_host[~inside]
    bad = np.count_nonzero(outside != sentinel)
    assert bad == 0, f"{what}: {bad} writes outside C's {rows} x {cols} window"
