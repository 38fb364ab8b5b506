"""Inputs of the exhaustive (w, s) sweeps (test infrastructure).

A stored scale is an outcome of the quantizer, not an input: it follows from
the group's extremes (s16 = fp16(fl32(fl32(mx - mn) / qmax))).  To put every
positive fp16 scale through the quantizer, each scale is realized by a pair
of extremes found on the oracle (oracle.rtn_scale_zero decides which pair
gives which stored scale), and the group's other entries run through every
fp16 value between the two extremes.

Nothing here computes a code: the expected codes, scales and zero points are
the oracle's, and the generator only chooses masters.
"""
import numpy as np

import oracle

F16 = np.float16
FP16_MAX_BITS = 0x7BFF                      # 65504


def every_finite_fp16():
    """All 63,488 finite fp16 values, in bit-pattern order (+0 ... 65504,
    -0 ... -65504)."""
    v = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(F16)
    return v[np.isfinite(v)]


def every_positive_fp16():
    """All 31,743 positive finite fp16 values (subnormals included)."""
    return np.arange(1, 0x7C00, dtype=np.uint32).astype(np.uint16).view(F16)


def _from_bits(b):
    return np.asarray(b, np.int64).astype(np.uint16).view(F16)


def realize_scales(scales, bits):
    """Extremes (mn <= 0 <= mx, fp16) whose group the oracle gives exactly
    the stored scale s, for each s in `scales`: a search around
    mn = -qmax*s/2, mx = qmax*s + mn over +-6 fp16 steps of each.
    Returns (found bool [S], mn fp16 [S], mx fp16 [S])."""
    scales = np.asarray(scales, F16)
    qmax = (1 << bits) - 1
    s64 = scales.astype(np.float64)
    a_bits = np.minimum(np.minimum(qmax * s64 / 2, 65504.0).astype(F16).view(np.uint16)
                        .astype(np.int64), FP16_MAX_BITS)
    a0 = _from_bits(a_bits).astype(np.float64)
    b_bits = np.minimum(np.minimum(qmax * s64 - a0, 65504.0).astype(F16).view(np.uint16)
                        .astype(np.int64), FP16_MAX_BITS)
    found = np.zeros(scales.size, bool)
    mn = np.zeros(scales.size, F16)
    mx = np.zeros(scales.size, F16)
    want = scales.view(np.uint16)
    for da in range(-6, 7):
        for db in range(-6, 7):
            A = _from_bits(np.clip(a_bits + da, 0, FP16_MAX_BITS))
            B = _from_bits(np.clip(b_bits + db, 0, FP16_MAX_BITS))
            s16, _ = oracle.rtn_scale_zero(np.stack([-A, B], axis=1), bits, 2)
            hit = ~found & (s16[:, 0].view(np.uint16) == want)
            mn[hit], mx[hit] = -A[hit], B[hit]
            found |= hit
    return found, mn, mx


def values_between(mn, mx):
    """Number of fp16 values in [mn, mx] for mn <= 0 <= mx, counting -0 and
    +0 both."""
    neg = mn.view(np.uint16).astype(np.int64) - 0x8000 + 1
    pos = mx.view(np.uint16).astype(np.int64) + 1
    return neg + pos


def quantizer_groups(mn, mx):
    """Groups of 64 masters for scales with extremes (mn[i], mx[i]): every
    fp16 value in [mn[i], mx[i]], 62 to a group, the two extremes in every
    group (so each group has that stored scale), padded with +0; each
    group's 64 entries are rotated by the group's index so the extremes
    visit every column.  Returns (W fp16 [R, 64], scale index of each row)."""
    mn = np.asarray(mn, F16)
    mx = np.asarray(mx, F16)
    cn = mn.view(np.uint16).astype(np.int64) - 0x8000 + 1     # -0 ... mn
    n_vals = values_between(mn, mx)
    groups = (n_vals + 61) // 62
    R = int(groups.sum())
    sidx = np.repeat(np.arange(mn.size), groups)
    row_in_scale = np.arange(R) - np.repeat(np.cumsum(groups) - groups, groups)
    k = row_in_scale[:, None] * 62 + np.arange(62)[None, :]        # value index in its scale
    cn_r = cn[sidx][:, None]
    vb = np.where(k < cn_r, 0x8000 + k, k - cn_r)
    vb = np.where(k < n_vals[sidx][:, None], vb, 0)                # padding: +0
    full = np.empty((R, 64), np.uint16)
    full[:, 0] = mn.view(np.uint16)[sidx]
    full[:, 1] = mx.view(np.uint16)[sidx]
    full[:, 2:] = vb.astype(np.uint16)
    shift = np.arange(R) % 64
    cols = (np.arange(64)[None, :] - shift[:, None]) % 64
    return np.take_along_axis(full, cols, axis=1).view(F16), sidx


def chunks_by_count(counts, target):
    """Consecutive index ranges [a, b) whose counts sum to about `target`."""
    out, a, acc = [], 0, 0
    for i, c in enumerate(np.asarray(counts).tolist()):
        acc += c
        if acc >= target:
            out.append((a, i + 1))
            a, acc = i + 1, 0
    if a < len(counts):
        out.append((a, len(counts)))
    return out
