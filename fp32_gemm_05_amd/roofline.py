"""Work and traffic counts of one SGEMM call, and the MI355X peaks they are priced against.

These are the measurement conventions of the bench and the profiling summaries:

* FLOPs: 2*M*N*K -- one multiply and one add per (i, j, k) ("SGEMM CUDA kernel (First
  Half)", "Part 4: Switching to Outer Product"); the alpha/beta epilogue is not counted.
* Algorithmic bytes: the compulsory traffic, each operand read once and C written once:
  4*(M*K + K*N + M*N), plus 4*M*N for the read of C when beta != 0.
* Panel read bytes: what a BM x BN output tiling reads from global memory when every tile
  streams its own A and B panels, K*(1/BM + 1/BN) values per output element ("1D Register
  Tiling: One Thread, TM Outputs", "The Arithmetic").  Where these re-reads are served (L2,
  Infinity Cache, HBM) is what the traffic counters measure.
"""
from __future__ import annotations

FP32_PEAK_TFLOPS = 157.3       # MI355X dense FP32 matrix (MFMA): 256 CUs x 2.4 GHz x 256 FLOP/clk
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X FP32 vector: 256 CUs x 2.4 GHz x 256 FLOP/clk
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E


def gemm_flops(M: int, N: int, K: int) -> float:
    return 2.0 * M * N * K


def algorithmic_bytes(M: int, N: int, K: int, beta: float) -> float:
    return 4.0 * (M * K + K * N + (2 if beta != 0 else 1) * M * N)


def panel_read_bytes(M: int, N: int, K: int, BM: int, BN: int) -> float:
    return 4.0 * M * N * K * (1.0 / BM + 1.0 / BN)


def tflops(M: int, N: int, K: int, ms: float) -> float:
    """TFLOP/s of one call of M x N x K that took ``ms`` milliseconds."""
    return gemm_flops(M, N, K) / (ms * 1e-3) / 1e12
