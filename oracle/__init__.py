"""fp64 CPU oracle for the fused GEMM + reduce-scatter share (test infrastructure only)."""
