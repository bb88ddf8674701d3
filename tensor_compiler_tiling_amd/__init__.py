"""tensor_compiler_tiling_amd -- NCHW conv2d (implicit GEMM on MI355X matrix
cores, split reduction, fused per-channel epilogue), per-channel broadcast and
a tile-config search, behind the C ABI in include/convtile.h.

Importing the package loads nothing; ``convtile`` loads libconvtile.so on
first use and raises if it is not built.
"""
__all__ = ["convtile", "workloads"]
