"""qlin on MI355X: fused dequantize-matmul over group-wise affine low-bit weights.

The computation lives in libqlin.so (HIP kernels for gfx950 behind the C ABI in
include/qlin.h); this package is its Python binding.
"""
from .qlin import (  # noqa: F401
    FMT_FP16_MASTER, FMT_PACKED, EXPORTS, LIB_PATH, QWeight, QlinError, embed_rows, gemm,
    gemm_multi, gemv,
    gemv_multi, gemv_swiglu, library, master_weight, meta_entries, packed_bytes, quantize,
    quantize_batch, workspace,
)
