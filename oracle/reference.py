"""Oracle for group-wise affine low-bit weights and the dequantize-matmul.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) may import or call this module; only ``tests/``, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` do.  It
shares no code, constant or table with the HIP path.

Plain, slow, obviously correct NumPy.  The quantizer arithmetic is pinned to
IEEE binary32 (every operand is ``np.float32`` so NumPy never promotes), the
dequantized weights and the matmul are computed in binary64.

What the method computes (sources: the Bitcrush README, sections "The
machine" and "Under the hood"; the Enargeia page, section "Run it"):

* Weights W are [N, K], N output features, K the reduction axis.  They are
  split along K into groups of 64 consecutive weights of one row ("SMART"),
  or one group per output row ("NAIVE", one scale per output channel).
* Each group gets one scale and one zero point.  Its codes are round-to-
  nearest: q = clamp(round(w / scale) + zero, 0, 2^bits - 1).
* A code is used as the weight scale * (q - zero); the matmul accumulates
  x * that value.  The fused form (Bitcrush's matmul_q) does the rounding
  inline from fp16 master weights; the packed form reads stored codes.

Where the pages leave a step open, the reading taken is stated at the step.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
# Every width of the lever (Bitcrush README, "The machine": the lever runs
# from 16 bits down to 2) has the same quantizer arithmetic and a packed-code
# layout (layout.py).
SUPPORTED_BITS = (2, 3, 4, 5, 6, 7, 8)
LEVER_BITS = (2, 3, 4, 5, 6, 7, 8)


def qmax_for(bits: int) -> int:
    """Largest code at ``bits`` bits (codes are unsigned, 0..2^bits-1)."""
    if bits not in LEVER_BITS:
        raise ValueError(f"bits must be one of {LEVER_BITS}, got {bits}")
    return (1 << bits) - 1


def _check_master(w16: np.ndarray, group: int) -> tuple[int, int, int]:
    if w16.dtype != np.float16 or w16.ndim != 2:
        raise TypeError("master weights must be a 2-D float16 array [N, K]")
    n, k = w16.shape
    if group <= 0 or k % group != 0:
        raise ValueError(f"K={k} is not a multiple of the group size {group}")
    if not np.all(np.isfinite(w16)):
        # The pages never define non-finite masters; the oracle refuses them.
        raise ValueError("master weights must be finite")
    return n, k, k // group


def rtn_scale_zero(w16: np.ndarray, bits: int, group: int):
    """Per-group scale (fp16) and zero point (uint8) by round-to-nearest.

    Bitcrush, "Under the hood": a separate kernel precomputes a scale and a
    zero per group before the fused matmul runs.  "The machine", NAIVE/SMART:
    the group is 64 weights along K (``group=64``) or the whole row
    (``group=K``).  Readings (the pages do not fix the arithmetic):

    1. mn, mx are the group's min and max, converted exactly to binary32.
    2. d = fl32(mx - mn); s32 = fl32(d / qmax) with IEEE division; the stored
       scale is s16 = fp16(s32) rounded to nearest-even; s = fp32(s16).
    3. zero = clamp(rint(fl32(-mn / s)), 0, qmax), with rint rounding ties to
       even and s the *stored* fp16 scale, so that the zero point and the
       codes use the same scale as the dequantizer.
    4. A group whose stored scale is 0 (all values equal, or d / qmax below
       the smallest fp16 subnormal) keeps scale 0 and zero 0; every code is
       0 and every dequantized weight is 0.

    Returns ``(scale16 float16 [N, G], zero uint8 [N, G])``.
    """
    n, k, g = _check_master(w16, group)
    qmax = F32(qmax_for(bits))
    wg = w16.astype(F32).reshape(n, g, group)
    mn = wg.min(axis=2)
    mx = wg.max(axis=2)
    d = (mx - mn).astype(F32)
    s32 = (d / qmax).astype(F32)
    s16 = s32.astype(np.float16)
    s = s16.astype(F32)
    degenerate = s16 == 0
    safe_s = np.where(degenerate, F32(1), s).astype(F32)
    zr = np.rint((-mn).astype(F32) / safe_s).astype(F32)
    z = np.clip(zr, F32(0), qmax)
    z = np.where(degenerate, F32(0), z)
    s16 = np.where(degenerate, np.float16(0), s16).astype(np.float16)
    return s16, z.astype(np.uint8)


def rtn_codes(w16: np.ndarray, scale16: np.ndarray, zero: np.ndarray,
              bits: int, group: int) -> np.ndarray:
    """Round-to-nearest codes of every weight, given its group's scale/zero.

    q = clamp(rint(fl32(w / s)) + zero, 0, qmax), with rint rounding ties to
    even (the pages only say "round-to-nearest"; binary round-half-even is
    the IEEE default).  The integer zero is added after rounding, and the
    clamp is applied in float before the conversion to an integer.  A group
    with scale 0 gets code 0 everywhere.  Returns uint8 [N, K].
    """
    n, k, g = _check_master(w16, group)
    qmax = F32(qmax_for(bits))
    w = w16.astype(F32).reshape(n, g, group)
    s = scale16.astype(np.float16).astype(F32).reshape(n, g, 1)
    z = zero.astype(F32).reshape(n, g, 1)
    degenerate = s == 0
    safe_s = np.where(degenerate, F32(1), s).astype(F32)
    t = np.rint(w / safe_s).astype(F32)
    q = np.clip((t + z).astype(F32), F32(0), qmax)
    q = np.where(degenerate, F32(0), q)
    return q.astype(np.uint8).reshape(n, k)


def quantize(w16: np.ndarray, bits: int, group: int):
    """Scale/zero precompute, then codes: ``(codes u8 [N,K], scale16, zero)``."""
    s16, z = rtn_scale_zero(w16, bits, group)
    return rtn_codes(w16, s16, z, bits, group), s16, z


def dequantize(codes: np.ndarray, scale16: np.ndarray, zero: np.ndarray,
               group: int) -> np.ndarray:
    """w_hat = scale * (q - zero) in binary64 (exact: an fp16 scale times an
    integer of at most 9 bits).  Enargeia, "Run it": the code is turned back
    into a weight this way and never stored in that form."""
    n, k = codes.shape
    g = k // group
    q = codes.astype(np.int64).reshape(n, g, group)
    z = zero.astype(np.int64).reshape(n, g, 1)
    s = scale16.astype(np.float16).astype(np.float64).reshape(n, g, 1)
    return (s * (q - z).astype(np.float64)).reshape(n, k)


def matmul_ref(x16: np.ndarray, w_hat: np.ndarray) -> np.ndarray:
    """Y = X @ W_hat^T with X (fp16) and W_hat converted exactly to binary64.

    x16 is [M, K] (or [K] for the M=1 decode form); returns [M, N] / [N]."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float64)
    return x @ np.asarray(w_hat, dtype=np.float64).T


def tolerance_scale(x16: np.ndarray, w_hat: np.ndarray) -> float:
    """T = max over outputs of sum_k |x_k * w_hat_k| (binary64).

    A GPU result Y passes when max |Y - Y_ref| <= 1e-3 * T: the bound covers
    the matmul arithmetic (rounding of the accumulation and of the operands),
    not the quantization error, which both sides share."""
    x = np.abs(np.asarray(x16, dtype=np.float16).astype(np.float64))
    return float(np.max(x @ np.abs(np.asarray(w_hat, np.float64)).T))


def fused_weights(w16: np.ndarray, scale16: np.ndarray, zero: np.ndarray,
                  bits: int, group: int) -> np.ndarray:
    """The weights the fused quantize-dequantize matmul multiplies by.

    Bitcrush, "Under the hood" (matmul_q): the fp16 master is re-quantized
    with the precomputed scale/zero as it is read, then dequantized; no code
    is stored.  bits=16 is the unquantized end of the lever: w itself."""
    if bits == 16:
        return np.asarray(w16, dtype=np.float16).astype(np.float64)
    return dequantize(rtn_codes(w16, scale16, zero, bits, group),
                      scale16, zero, group)


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), in binary64.

    The activation of the gated MLP that follows the gate and up projections
    (Bitcrush README, "Under the hood": the SwiGLU kernel of the decode path).
    exp(-g) overflows to inf for g < -709; g / inf is then the correct -0."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ref(x16: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """h = silu(x . W_gate^T) * (x . W_up^T): the two decode GEMVs that share
    the MLP input, combined elementwise (binary64 throughout)."""
    return silu(matmul_ref(x16, w_gate)) * matmul_ref(x16, w_up)


# Largest slope of silu: silu'(g) = s(g) (1 + g (1 - s(g))), s the logistic
# function, peaks at 1.0998 near g = 2.40; 1.1 bounds it.
SILU_SLOPE_MAX = 1.1


def swiglu_tolerance(x16: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray,
                     rel: float = 1e-3, fp32_rel: float = 4e-6) -> np.ndarray:
    """Per-output bound on |h_gpu - h_ref| implied by the GEMV tolerance.

    The GEMV contract bounds the gate and up sums by eg = rel * T_gate and
    eu = rel * T_up (T = max_row sum |x w|).  With |silu'| <= 1.1:
        |silu(g + dg)(u + du) - silu(g) u|
            <= 1.1 eg (|u| + eu) + |silu(g)| eu,
    and the fp32 evaluation of silu and of the product adds at most
    fp32_rel * |h| (a few ulp of binary32)."""
    g = matmul_ref(x16, w_gate)
    u = matmul_ref(x16, w_up)
    eg = rel * tolerance_scale(x16, w_gate)
    eu = rel * tolerance_scale(x16, w_up)
    prop = SILU_SLOPE_MAX * eg * (np.abs(u) + eu) + np.abs(silu(g)) * eu
    return prop * (1.0 + fp32_rel) + fp32_rel * np.abs(silu(g) * u)
