"""The fp16 range of the GEMM's weight operand, pinned on the oracle.

The prefill GEMM feeds the matrix cores with each dequantized weight
w_hat = s * (q - z) rounded once to fp16; a value of magnitude >= 65520 rounds
to infinity.  For a group whose masters all satisfy |w| <= L, the largest
|w_hat| is s * max(z, qmax - z), and it grows with the group's extremes, so the
worst case has one extreme at +L or -L and the other anywhere in [-L, L]
(the largest |w_hat| of a group is that of one of its extremes).  The
admissible magnitudes below (the largest multiple of 32 -- fp16's spacing
there -- for which no such group overflows) are checked here by brute force
over every fp16 value of the other extreme, with the oracle's own codes, and
shown to be tight: 32 more makes some group overflow.  Masters beyond them are handled by the GEMM
kernels (a block whose operand would overflow is evaluated with the operand
scaled by 2^-8 and the product scaled back), so they are not refused.
"""
import numpy as np
import pytest

import oracle

# largest |w| (a multiple of 32) with every w_hat finite in fp16, per width
ADMISSIBLE = {2: 49120, 3: 57312, 4: 61408, 5: 63456, 6: 64480, 7: 64992, 8: 65248}

POS = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)   # every finite fp16 >= 0


def _groups(L):
    """Every group with one extreme at +L or -L and the other at any fp16
    value of the opposite sign (the rest of the group 0)."""
    L = np.float16(L)
    a = POS[POS <= L]
    g = np.zeros((2 * a.size, 64), np.float16)
    g[: a.size, 0] = -a
    g[: a.size, 1] = L
    g[a.size:, 0] = -L
    g[a.size:, 1] = a
    return g


def _w_hat(g, bits):
    codes, s16, z = oracle.quantize(g, bits, 64)
    return oracle.dequantize(codes, s16, z, 64)


def worst_w_hat(bits, L):
    """The largest |w_hat| over those groups, from the oracle's own codes."""
    return float(np.max(np.abs(_w_hat(_groups(L), bits))))


@pytest.mark.parametrize("bits", sorted(ADMISSIBLE))
def test_admissible_master_range_is_tight(bits):
    L = ADMISSIBLE[bits]
    assert worst_w_hat(bits, L) < 65520            # rounds to at most 65504
    assert worst_w_hat(bits, L + 32) >= 65520      # rounds to infinity


def worst_group(bits, L):
    """The group of _groups(L) with the largest |w_hat|."""
    g = _groups(L)
    return g[np.argmax(np.max(np.abs(_w_hat(g, bits)), axis=1))][None, :]


@pytest.mark.parametrize("bits", sorted(ADMISSIBLE))
def test_extreme_group_dequantizes_past_fp16(bits):
    """Finite masters near the ends of the fp16 range can dequantize to
    weights that fp16 cannot hold -- the case the GEMM kernels handle: the
    worst group with extremes up to 65504 has a code whose w_hat, exact in
    binary64, rounds to infinity in fp16."""
    w = worst_group(bits, 65504)
    codes, s16, z = oracle.quantize(w, bits, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    assert np.all(np.isfinite(what))               # exact in binary64
    assert np.max(np.abs(what)) >= 65520
    with np.errstate(over="ignore"):
        assert not np.all(np.isfinite(what.astype(np.float16)))


def test_formula_bound_is_below_the_scan():
    """The closed-form bound |w_hat| <= L (1 + 2^-10 + (1 + 2^-11) / qmax)
    (one extreme, plus the fp16 rounding of the scale times qmax, plus half a
    step from rounding the zero point) implies the scanned values are safe
    margins: the largest L it admits is at most the tight value."""
    for bits, L in ADMISSIBLE.items():
        qmax = (1 << bits) - 1
        formula_L = 65520 / (1 + 2 ** -10 * 1.0001 + (1 + 2 ** -11) / qmax)
        assert formula_L <= L + 32
        assert worst_w_hat(bits, np.floor(formula_L / 32) * 32) < 65520
