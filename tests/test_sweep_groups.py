"""The sweep inputs (tests/sweep_groups.py) do what the GPU sweep relies on:
every reachable stored scale is realized, and the groups hold every fp16
value between their extremes with that stored scale (checked on the oracle)."""
import numpy as np
import pytest

import oracle
import sweep_groups as sg


def test_every_fp16_counts():
    assert sg.every_finite_fp16().size == 63488
    s = sg.every_positive_fp16()
    assert s.size == 31743 and np.all(s > 0) and np.all(np.isfinite(s))


@pytest.mark.parametrize("bits,top", [(2, 43680.0), (8, 514.0)])
def test_every_reachable_scale_is_realized(bits, top):
    """d = fl32(mx - mn) <= 131008, so s32 <= 131008 / qmax and the stored
    scale is at most fp16 of that (43680 at 2 bits, 514 at 8): every
    positive fp16 up to there is realized, and nothing above."""
    s = sg.every_positive_fp16()
    found, mn, mx = sg.realize_scales(s, bits)
    sf = s.astype(np.float64)
    assert float(np.float16(np.float32(131008) / np.float32((1 << bits) - 1))) == top
    assert np.all(found == (sf <= top))
    assert np.all(mn[found] <= 0) and np.all(mx[found] >= 0)
    s16, _ = oracle.rtn_scale_zero(np.stack([mn[found], mx[found]], axis=1), bits, 2)
    assert np.array_equal(s16[:, 0].view(np.uint16), s[found].view(np.uint16))


@pytest.mark.parametrize("bits", [2, 8])
def test_groups_cover_the_range_with_the_stored_scale(bits):
    s = sg.every_positive_fp16()
    found, mn, mx = sg.realize_scales(s, bits)
    sel = np.flatnonzero(found)[::1499]
    W, sidx = sg.quantizer_groups(mn[sel], mx[sel])
    s16, _ = oracle.rtn_scale_zero(W, bits, 64)
    assert np.array_equal(s16[:, 0].view(np.uint16), s[sel][sidx].view(np.uint16))
    for i, j in enumerate(sel):
        got = np.unique(W[sidx == i].view(np.uint16))
        lo, hi = mn[j].view(np.uint16), mx[j].view(np.uint16)
        want = np.union1d(np.arange(0x8000, int(lo) + 1), np.arange(0, int(hi) + 1))
        assert np.array_equal(got, want.astype(np.uint16))


def test_chunks_by_count():
    assert sg.chunks_by_count([5, 5, 5, 1], 10) == [(0, 2), (2, 4)]
    assert sg.chunks_by_count([20, 1], 10) == [(0, 1), (1, 2)]
