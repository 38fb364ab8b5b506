"""Pins of the oracle's tolerance scale T and of its fused-weight route.

T = max over outputs (m, n) of sum_k |x[m,k] * w_hat[n,k]| is the yardstick of
every matmul parity check (max |Y - Y_ref| <= 1e-3 * T).  Here T is computed
independently, in exact rational arithmetic, and compared for equality with
``oracle.tolerance_scale`` on inputs where binary64 represents every partial
sum exactly (small dyadic values), so that any slip in the formula -- a sum
where the maximum belongs, a missing absolute value on x or on w_hat, the
absolute value taken after summing, the maximum taken over one axis only, a
transposed operand -- changes the result.
"""
from fractions import Fraction
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def exact_T(x, w):
    x = np.atleast_2d(x)
    best = None
    for m in range(x.shape[0]):
        for n in range(w.shape[0]):
            t = sum(abs(Fraction(float(x[m, k])) * Fraction(float(w[n, k])))
                    for k in range(w.shape[1]))
            best = t if best is None or t > best else best
    return best


def dyadic(rng, shape, den=64, lo=-40, hi=41):
    """Signed multiples of 1/den: every product and partial sum below is
    exact in binary64, so equality with the rational T is exact."""
    return rng.integers(lo, hi, size=shape).astype(np.float64) / den


def test_single_output_hand_value():
    # x = (1, -2, 3), w = (-4, 5, -6): sum |x w| = 4 + 10 + 18 = 32
    x = np.array([1, -2, 3], dtype=np.float16)
    w = np.array([[-4.0, 5.0, -6.0]])
    assert oracle.tolerance_scale(x, w) == 32.0
    # with |.| after the sum it would be |-4 - 10 - 18| = 32 too, so also a
    # mixed-sign case: x = (1, 2, 3), w = (-4, 5, -6): 4 + 10 + 18 = 32,
    # while |sum x w| = |-4 + 10 - 18| = 12
    x = np.array([1, 2, 3], dtype=np.float16)
    assert oracle.tolerance_scale(x, w) == 32.0


@pytest.mark.parametrize("m,n,k,seed", [(1, 5, 64, 0), (3, 4, 64, 1), (4, 7, 128, 2),
                                        (2, 9, 192, 3), (5, 3, 64, 4)])
def test_equals_exact_rational(m, n, k, seed):
    rng = np.random.default_rng(seed)
    x = dyadic(rng, (m, k), den=16).astype(np.float16)
    w = dyadic(rng, (n, k))
    assert np.array_equal(x.astype(np.float64), dyadic(np.random.default_rng(seed), (m, k), 16))
    T = exact_T(x, w)
    assert Fraction(oracle.tolerance_scale(x, w)) == T
    if m == 1:   # the decode form takes x as a vector
        assert Fraction(oracle.tolerance_scale(x[0], w)) == T


def test_max_output_is_not_the_largest_weight_row():
    """Row 0 holds the largest |w| but x is zero where it sits; row 1's
    moderate weights meet large |x|.  The maximum is over outputs of the
    whole sum, not over single weights or single activations."""
    k = 64
    x = np.zeros((2, k), dtype=np.float16)
    x[0, 1:] = np.float16(-2)     # signed, large
    x[1, 1:] = np.float16(0.5)
    w = np.zeros((3, k))
    w[0, 0] = 1000.0              # the largest |w|, multiplied by x = 0
    w[0, 1] = 1.0
    w[1, 1:] = np.where(np.arange(1, k) % 2 == 0, 3.0, -3.0)   # alternating signs
    w[2, 1:] = 0.25
    T = exact_T(x, w)
    # the maximum is at (m = 0, n = 1): 63 * 2 * 3 = 378
    assert T == 378
    assert oracle.tolerance_scale(x, w) == 378.0
    # a sum over outputs in place of the maximum would give
    # (2 + 378 + 31.5) + (0.5 + 94.5 + 7.875) = 514.375
    assert oracle.tolerance_scale(x, w) != 514.375


def test_max_over_both_axes():
    """The largest output sits at m > 0 and n > 0: a maximum over only one
    axis (or only the first row of X) misses it."""
    rng = np.random.default_rng(8)
    x = dyadic(rng, (4, 64), den=16).astype(np.float16)
    w = dyadic(rng, (6, 64))
    x[3] = np.float16(4) * np.sign(x[3]).astype(np.float16)
    w[5] = 2.0 * np.sign(w[5])
    T = exact_T(x, w)
    assert Fraction(oracle.tolerance_scale(x, w)) == T
    per_out = np.abs(x.astype(np.float64)) @ np.abs(w).T
    assert np.unravel_index(np.argmax(per_out), per_out.shape) == (3, 5)


def _load(path):
    d = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            key, val = line.split(":", 1)
            d[key.strip()] = val.split()

    def expand(tokens, cast):
        out = []
        for t in tokens:
            if "*" in t:
                v, c = t.split("*")
                out += [cast(v)] * int(c)
            else:
                out.append(cast(t))
        return out
    return (int(d["bits"][0]), int(d["group"][0]), np.array(expand(d["w"], float)),
            int(d["scale16"][0], 16), int(d["zero"][0]), np.array(expand(d["what"], float)))


@pytest.mark.parametrize("name", ["example_a.txt", "example_b.txt", "example_d.txt",
                                  "example_f.txt", "example_g.txt", "example_h.txt",
                                  "example_i.txt"])
def test_fused_weights_reproduce_hand_worked_values(name):
    """The fused route (re-round the fp16 master with a given scale and zero,
    then dequantize) gives the hand-worked dequantized weights when it is
    handed the hand-worked scale and zero -- not the oracle's own."""
    bits, group, w, s_bits, z, what = _load(os.path.join(GOLDEN, name))
    w16 = w.astype(np.float16).reshape(1, -1)
    s16 = np.array([[s_bits]], dtype=np.uint16).view(np.float16)
    zero = np.array([[z]], dtype=np.uint8)
    got = oracle.fused_weights(w16, s16, zero, bits, group)
    assert np.array_equal(got[0], what)
