"""Oracle vs exact rational arithmetic on small inputs.

An independent re-statement of the quantizer with ``fractions.Fraction``:
binary32/binary16 rounding is done here by hand (round to nearest, ties to
even, with subnormals), so a wrong dtype, a wrong rounding mode, a dropped
term or a transposed operand in the NumPy oracle shows up as a mismatch.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def _round_binary(x: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Round x to the nearest binary float with ``mant_bits`` fraction bits and
    minimum normal exponent ``emin`` (ties to even; no overflow handling)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - mant_bits)
    q, r = divmod(a, ulp)
    q = int(q)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return sign * q * ulp


def f32(x: Fraction) -> Fraction:
    return _round_binary(x, 23, -126)


def f16(x: Fraction) -> Fraction:
    return _round_binary(x, 10, -14)


def rint_even(x: Fraction) -> int:
    f = x.numerator // x.denominator
    r = x - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def exact_quantize(w16: np.ndarray, bits: int, group: int):
    qmax = (1 << bits) - 1
    n, k = w16.shape
    codes = np.zeros((n, k), dtype=np.int64)
    scales = np.zeros((n, k // group), dtype=object)
    zeros = np.zeros((n, k // group), dtype=np.int64)
    for r in range(n):
        for g in range(k // group):
            vals = [Fraction(float(v)) for v in w16[r, g * group:(g + 1) * group]]
            mn, mx = min(vals), max(vals)
            s = f16(f32(f32(mx - mn) / qmax))
            if s == 0:
                scales[r, g] = Fraction(0)
                continue
            z = min(max(rint_even(f32(-mn / s)), 0), qmax)
            scales[r, g] = s
            zeros[r, g] = z
            for i, v in enumerate(vals):
                codes[r, g * group + i] = min(max(rint_even(f32(v / s)) + z, 0), qmax)
    return codes, scales, zeros


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, 128])
def test_quantizer_matches_exact_arithmetic(bits, group):
    rng = np.random.default_rng(100 + bits)
    w16 = np.concatenate([synth.master_weights(rng, 3, 128),
                          synth.edge_groups(bits, rng, n_rows=3, k=128)])
    codes, s16, z = oracle.quantize(w16, bits, group)
    ecodes, es, ez = exact_quantize(w16, bits, group)
    for r in range(w16.shape[0]):
        for g in range(w16.shape[1] // group):
            assert Fraction(float(s16[r, g])) == es[r, g]
            assert int(z[r, g]) == ez[r, g]
    assert np.array_equal(codes.astype(np.int64), ecodes)


def test_matmul_matches_exact_sums():
    rng = np.random.default_rng(5)
    for bits in (2, 4):
        w16 = synth.master_weights(rng, 7, 128)
        x16 = synth.activations(rng, 3, 128)
        codes, s16, z = oracle.quantize(w16, bits, 64)
        what = oracle.dequantize(codes, s16, z, 64)
        y = oracle.matmul_ref(x16, what)
        t = oracle.tolerance_scale(x16, what)
        for m in range(3):
            for n in range(7):
                exact = sum(Fraction(float(x16[m, kk])) * Fraction(float(what[n, kk]))
                            for kk in range(128))
                tabs = sum(abs(Fraction(float(x16[m, kk])) * Fraction(float(what[n, kk])))
                           for kk in range(128))
                assert abs(Fraction(float(y[m, n])) - exact) <= Fraction(128, 2 ** 52) * tabs
                assert float(tabs) <= t * (1 + 1e-15)
        # the dequantized weights themselves are exact: s * (q - z)
        for n in range(7):
            for kk in range(0, 128, 9):
                g = kk // 64
                assert Fraction(float(what[n, kk])) == Fraction(float(s16[n, g])) * (
                    int(codes[n, kk]) - int(z[n, g]))


def test_closed_forms():
    """One-hot x picks one column of W_hat exactly; x = 1 gives row sums; a
    group whose codes are all equal contributes s*(q - z)*sum(x)."""
    rng = np.random.default_rng(9)
    w16 = synth.master_weights(rng, 16, 256)
    codes, s16, z = oracle.quantize(w16, 4, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    for kk in (0, 63, 64, 200, 255):
        x = np.zeros(256, dtype=np.float16)
        x[kk] = 1
        assert np.array_equal(oracle.matmul_ref(x, what), what[:, kk])
    ones = np.ones(256, dtype=np.float16)
    rs = [sum(Fraction(float(v)) for v in what[n]) for n in range(16)]
    y = oracle.matmul_ref(ones, what)
    for n in range(16):
        assert abs(Fraction(float(y[n])) - rs[n]) <= Fraction(256, 2 ** 52) * sum(
            abs(Fraction(float(v))) for v in what[n])
    # constant-code group: codes forced equal
    c2 = codes.copy()
    c2[:, :64] = 11
    what2 = oracle.dequantize(c2, s16, z, 64)
    x = synth.activations(rng, 1, 256)[0]
    x[64:] = 0
    y2 = oracle.matmul_ref(x, what2)
    xs = float(np.sum(x[:64].astype(np.float64)))
    for n in range(16):
        expect = float(s16[n, 0]) * (11 - int(z[n, 0])) * xs
        assert abs(y2[n] - expect) <= 1e-12 * max(1.0, abs(expect))


def test_fused_weights_equal_packed_route_and_bits16_identity():
    rng = np.random.default_rng(11)
    w16 = synth.master_weights(rng, 8, 192)
    for bits in (2, 3, 4, 8):
        for group in (64, 192):
            codes, s16, z = oracle.quantize(w16, bits, group)
            assert np.array_equal(oracle.fused_weights(w16, s16, z, bits, group),
                                  oracle.dequantize(codes, s16, z, group))
    assert np.array_equal(oracle.fused_weights(w16, None, None, 16, 64),
                          w16.astype(np.float64))
