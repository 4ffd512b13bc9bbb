"""Seeded synthetic SGEMM workloads (shapes, scalars, value distributions).

This module only draws input matrices; it holds none of the GEMM arithmetic.
It is the one piece shared by the HIP path's tests and bench and by the oracle's
checks, so that both sides see the very same arrays.

The pages measure square 4096 x 4096 x 4096 products ("1D Register Tiling: One
Thread, TM Outputs", section "Mechanics"; "Global Memory Coalescing", section
"Mechanics") without stating their value distribution; the workloads below are
synthetic stand-ins with those shapes plus the ragged, small, large and skinny
shapes of the workload list.

Recipe (numpy PCG64, one generator per workload, draws in the order A, B, C):
  * "uniform": ``rng.uniform(-1, 1, shape).astype(float32)``
  * "normal":  ``rng.standard_normal(shape, dtype=float32)``
  * "int":     ``rng.integers(-2, 3, shape).astype(float32)``  (values -2..2)
C is drawn only when beta != 0; otherwise it is all zeros.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dist: str          # "uniform" | "normal" | "int"
    seed: int
    roofline: str = "compute"  # the roof the workload is reported against: "compute" or "hbm"

    def as_int(self) -> "Workload":
        """The integer-valued variant of this workload (same shape and scalars)."""
        return replace(self, name=self.name + "-int", dist="int", seed=self.seed + 1000)

    def describe(self) -> str:
        return (f"sgemm M={self.M} N={self.N} K={self.K} alpha={self.alpha:g} "
                f"beta={self.beta:g} dist={self.dist} seed={self.seed}")


# The workload list.  Seeds are fixed so that every run sees the same arrays.
WORKLOADS = {
    "square256": Workload("square256", 256, 256, 256, 1.0, 0.0, "uniform", 1001),
    "square1024_beta": Workload("square1024_beta", 1024, 1024, 1024, 1.0, 0.5, "uniform", 1003),
    "square4096": Workload("square4096", 4096, 4096, 4096, 1.0, 0.0, "uniform", 1004),
    "ragged3001x5003x777": Workload("ragged3001x5003x777", 3001, 5003, 777, 0.5, -1.5, "normal", 1005),
    "square8192": Workload("square8192", 8192, 8192, 8192, 1.0, 0.0, "uniform", 1006),
    # tall-skinny: one pass over a 256 MiB A, reported against the HBM roofline
    "skinny65536x64x1024": Workload("skinny65536x64x1024", 65536, 64, 1024, 1.0, 0.0, "uniform", 1007, "hbm"),
    # narrower still (N <= 32): a 512 MiB A streamed once; the 32-wide-tile class
    "narrow262144x32x512": Workload("narrow262144x32x512", 262144, 32, 512, 1.0, 0.0, "uniform", 1008, "hbm"),
}

# The headline workload that the bench times.
HEADLINE = "square4096"


def _draw(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, shape).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "int":
        return rng.integers(-2, 3, shape).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(w: Workload, M=None, N=None, K=None, dist=None, seed=None, beta=None):
    """Draw (A, B, C) as C-contiguous float32 arrays for workload ``w``.

    Shape, distribution, seed and beta may be overridden (used for reduced-size
    parity cases that keep a workload's character).
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    dist = w.dist if dist is None else dist
    seed = w.seed if seed is None else seed
    beta = w.beta if beta is None else beta
    rng = np.random.default_rng(seed)
    A = _draw(rng, dist, (M, K))
    B = _draw(rng, dist, (K, N))
    if beta != 0.0:
        C = _draw(rng, dist, (M, N))
    else:
        C = np.zeros((M, N), dtype=np.float32)
    return A, B, C


def padded(x: np.ndarray, pad: int, fill=np.nan) -> np.ndarray:
    """Return a view of ``x`` whose rows sit in a wider buffer (row stride = cols + pad).

    The extra columns hold ``fill`` (NaN by default), so a kernel that reads or
    writes past a row's end is caught.
    """
    rows, cols = x.shape
    buf = np.full((rows, cols + pad), fill, dtype=x.dtype)
    buf[:, :cols] = x
    return buf[:, :cols]


def sample_points(M: int, N: int, n_random: int, seed: int, tile: int = 256):
    """Output coordinates for sampled full-size checks.

    Returns int64 arrays (I, J): ``n_random`` uniform points plus every corner
    and the first/last rows and columns at tile-boundary offsets, so that edge
    tiles and the ragged tails are always covered.
    """
    rng = np.random.default_rng(seed)
    I = list(rng.integers(0, M, n_random))
    J = list(rng.integers(0, N, n_random))
    edge_r = sorted({0, 1, M // 2, M - 2, M - 1} | {min(M - 1, t) for t in range(tile - 1, M, tile)})
    edge_c = sorted({0, 1, N // 2, N - 2, N - 1} | {min(N - 1, t) for t in range(tile - 1, N, tile)})
    edge_r = [r for r in edge_r if 0 <= r < M]
    edge_c = [c for c in edge_c if 0 <= c < N]
    for r in edge_r:
        for c in (0, N - 1, N // 2):
            I.append(r)
            J.append(c)
    for c in edge_c:
        for r in (0, M - 1, M // 2):
            I.append(r)
            J.append(c)
    return np.asarray(I, dtype=np.int64), np.asarray(J, dtype=np.int64)
