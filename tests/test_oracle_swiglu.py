"""Pins for the oracle's gated-MLP combination h = silu(x.Wg^T) * (x.Wu^T).

silu is pinned by closed forms (sigmoid(ln 3) = 3/4 exactly, the odd-part
identity silu(x) - silu(-x) = x, the limits), the combination by a hand-built
one-hot case, and the derived tolerance by brute force over worst-case
perturbations of the two GEMV results."""
import numpy as np

import oracle


def test_silu_closed_forms():
    ln3 = np.log(3.0)
    # sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4;  sigmoid(-ln 3) = 1/4
    assert abs(oracle.silu(np.array(ln3)) - 0.75 * ln3) <= 1e-15
    assert abs(oracle.silu(np.array(-ln3)) + 0.25 * ln3) <= 1e-15
    assert oracle.silu(np.array(0.0)) == 0.0
    # odd-part identity: silu(x) - silu(-x) = x (sigmoid(-x) = 1 - sigmoid(x))
    x = np.random.default_rng(0).standard_normal(1000) * 5
    assert np.max(np.abs(oracle.silu(x) - oracle.silu(-x) - x)) <= 1e-13
    # limits: identity for large g, -0 (not nan) when exp(-g) overflows
    assert oracle.silu(np.array(40.0)) == 40.0
    big_neg = oracle.silu(np.array([-800.0, -1e300]))
    assert np.all(big_neg == 0.0) and not np.any(np.isnan(big_neg))


def test_silu_slope_bound():
    g = np.linspace(-20, 20, 400001)
    s = 1 / (1 + np.exp(-g))
    slope = s * (1 + g * (1 - s))
    assert slope.max() < oracle.SILU_SLOPE_MAX
    assert slope.max() > 1.0998     # the bound is tight, not a loose guess
    # finite differences of the oracle's silu agree with the analytic slope
    fd = np.diff(oracle.silu(g)) / np.diff(g)
    assert np.max(np.abs(fd - 0.5 * (slope[1:] + slope[:-1]))) < 1e-6


def test_swiglu_one_hot_case():
    ln3 = np.log(3.0)
    # x = e_0 selects column 0 of both weights: g = (ln 3, 0, -ln 3), u = (2, 5, 4)
    wg = np.zeros((3, 64)); wg[:, 0] = [ln3, 0.0, -ln3]
    wu = np.zeros((3, 64)); wu[:, 0] = [2.0, 5.0, 4.0]
    x = np.zeros(64, dtype=np.float16); x[0] = 1
    h = oracle.swiglu_ref(x, wg, wu)
    np.testing.assert_allclose(h, [1.5 * ln3, 0.0, -ln3], rtol=0, atol=1e-15)


def test_swiglu_tolerance_covers_worst_perturbations():
    rng = np.random.default_rng(3)
    n, k = 96, 256
    wg = rng.standard_normal((n, k)) * 0.05
    wu = rng.standard_normal((n, k)) * 0.05
    x = rng.standard_normal(k).astype(np.float16)
    h = oracle.swiglu_ref(x, wg, wu)
    bound = oracle.swiglu_tolerance(x, wg, wu)
    g = oracle.matmul_ref(x, wg)
    u = oracle.matmul_ref(x, wu)
    eg = 1e-3 * oracle.tolerance_scale(x, wg)
    eu = 1e-3 * oracle.tolerance_scale(x, wu)
    worst = np.zeros(n)
    for dg in np.linspace(-eg, eg, 21):
        for du in (-eu, 0.0, eu):
            worst = np.maximum(worst, np.abs(oracle.silu(g + dg) * (u + du) - h))
    assert np.all(worst <= bound)
    # and the bound is not vacuous: somewhere it is within 2x of the worst case
    # (elsewhere the global slope bound 1.1 exceeds the local slope of silu)
    assert np.min(bound / np.maximum(worst, 1e-300)) < 2.0
