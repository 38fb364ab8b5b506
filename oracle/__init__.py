"""CPU oracle for qlin: test infrastructure, never part of the product path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` import this package.  It imports nothing from the HIP library or
its binding, and they import nothing from it.
"""
from .reference import (  # noqa: F401
    SUPPORTED_BITS, LEVER_BITS, qmax_for, rtn_scale_zero, rtn_codes, quantize, dequantize,
    matmul_ref, tolerance_scale, fused_weights, silu, swiglu_ref, swiglu_tolerance,
    SILU_SLOPE_MAX,
)
from .layout import (  # noqa: F401
    TILE_ROWS, KBLOCK, words_per_block, code_bit_map, n_tiles, packed_words,
    pack_codes, unpack_codes, tile_meta, untile_meta,
)
