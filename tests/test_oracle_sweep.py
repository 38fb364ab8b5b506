"""Exhaustive code sweep over every finite fp16 weight and fp16 scale.

Pins the division step of the quantizer: for every finite fp16 w and every
positive finite fp16 s with |w/s| <= 512 (beyond that every code clamps),
rint(fl32(w / s)) -- the oracle's arithmetic -- equals the round-half-even of
the exact quotient.  The exact quotient is taken in binary64, which is exact
at the ties (k + 1/2 is representable) and far from every other half-integer
(an fp16/fp16 quotient that is not a tie is at least ~2^-22 relative away
from one, binary64 errs by 2^-53).

The same sweep checks the cheaper arithmetic a kernel may use instead of a
correctly rounded divide: t = fl32(w * fl32(1/s)), q0 = rint(t), and at an
exact tie (|w - q0*s| == s/2, an exact test) the even neighbour.  That this
agrees everywhere is what licenses it.

The default run takes every 7th scale (all weights); the full sweep is
marked slow.
"""
import numpy as np
import pytest


def _all_finite_fp16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


def _positive_scales():
    bits = np.arange(1, 0x7C00, dtype=np.uint32).astype(np.uint16)
    return bits.view(np.float16)


def _sweep(scales):
    w16 = _all_finite_fp16()
    w32 = w16.astype(np.float32)[None, :]
    w64 = w16.astype(np.float64)[None, :]
    bad_div = bad_rcp = ties = 0
    for i in range(0, scales.size, 48):
        s16 = scales[i:i + 48]
        s32 = s16.astype(np.float32)[:, None]
        s64 = s16.astype(np.float64)[:, None]
        ref = np.rint(w64 / s64)
        inrange = np.abs(w64 / s64) <= 512
        oq = np.rint(w32 / s32).astype(np.float64)
        bad_div += int(np.count_nonzero((oq != ref) & inrange))
        r32 = (np.float32(1) / s32).astype(np.float32)
        q0 = np.rint((w32 * r32).astype(np.float32)).astype(np.float64)
        e = w64 - q0 * s64                       # exact: fits in 24 bits here
        tie = np.abs(e) == s64 / 2
        kq = np.where(tie, np.rint(q0 + np.copysign(0.5, e)), q0)
        bad_rcp += int(np.count_nonzero((kq != ref) & inrange))
        ties += int(np.count_nonzero(tie & inrange))
    return bad_div, bad_rcp, ties


def test_code_sweep_sampled():
    bad_div, bad_rcp, ties = _sweep(_positive_scales()[::7])
    assert bad_div == 0
    assert bad_rcp == 0
    assert ties > 1000


@pytest.mark.slow
def test_code_sweep_full():
    bad_div, bad_rcp, ties = _sweep(_positive_scales())
    assert bad_div == 0
    assert bad_rcp == 0
    assert ties > 100000
