"""Measurement arithmetic used by the benchmark: throughput, exposed
communication fraction, and the per-tile overlap bound.

The formulas are the ones the ParallelKittens pages use to read their own
measurements ("ParallelKittens: Three Principles and Eight Primitives for
Multi-GPU Kernels", section 3 "Principle 2", and the summary page's section 3
"Scheduling Analysis", Table 3):

* a GEMM of shape M x N x K performs 2*M*N*K floating-point operations;
* the non-overlapped communication share of a fused kernel is
  (t_fused - t_gemm) / t_fused;
* one m x n output tile costs 2*m*n*K / R seconds of matrix-core time and
  s*m*n / B seconds of transfer, so transfer hides behind compute when
  K >= s*R / (2*B); the tile sides cancel.
"""
from __future__ import annotations

# MI355X published peaks used as roofline denominators.
PEAK_BF16_DENSE_FLOPS = 2.5e15       # dense bf16 MFMA, FLOP/s
PEAK_HBM_BYTES = 8.0e12              # HBM3E, bytes/s


def gemm_flops(M: int, N: int, K: int) -> float:
    return 2.0 * float(M) * float(N) * float(K)


def tflops(M: int, N: int, K: int, seconds: float) -> float:
    return gemm_flops(M, N, K) / seconds / 1e12


def exposed_fraction(t_fused: float, t_gemm: float) -> float:
    """Share of the fused time not hidden behind the GEMM."""
    return (t_fused - t_gemm) / t_fused


def overlap_threshold_k(s_bytes: float, R_flops: float, B_bytes: float) -> float:
    """Smallest K for which per-tile compute covers the per-tile transfer."""
    return s_bytes * R_flops / (2.0 * B_bytes)


def tile_compute_seconds(m: int, n: int, K: int, R_flops: float) -> float:
    return 2.0 * m * n * K / R_flops


def tile_transfer_seconds(m: int, n: int, s_bytes: float, B_bytes: float) -> float:
    return s_bytes * m * n / B_bytes
