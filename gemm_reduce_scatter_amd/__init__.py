"""One GPU's share of a tile-fused bf16 GEMM + reduce-scatter on MI355X (gfx950).

The compute path is the HIP library ``libpk_gemm_rs.so`` built from
``csrc/``; :mod:`gemm_reduce_scatter_amd.binding` marshals torch tensors into
its C entry points.  Importing the package does not load the library.
"""
__all__ = ["binding", "inputs", "metrics"]
