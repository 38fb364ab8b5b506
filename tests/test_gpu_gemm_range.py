"""GPU parity of the GEMMs at the ends of the fp16 range.

The GEMMs feed the matrix cores with s * (q - z) rounded to fp16.  Masters up
to the admissible magnitude of their width (test_oracle_gemm_range.ADMISSIBLE)
dequantize to fp16-finite operands; beyond it a dequantized weight can reach
65520 and fp16 cannot hold it, and the kernels then decode the tile with the
scale times 2^-8 and scale the sums back.  Both cases must stay finite and
within max |Y - Y_ref| <= 1e-3 * T of the oracle, for every width and every
kernel form (forced through the launch-shape override), and for the SwiGLU
pair's fp32 output.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from group_wise_bit_amd import qlin

from test_oracle_gemm_range import ADMISSIBLE, worst_group

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-3


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def masters(bits, L, n, k, seed):
    """N(0, 0.02) masters whose rows each carry, in one group, the group of
    extremes up to L with the largest dequantized weight (rows 0, 5, 70 and
    the last: different tiles, column halves and lanes)."""
    rng = np.random.default_rng(seed)
    w = synth.master_weights(rng, n, k)
    g = worst_group(bits, L)[0]
    for r, grp in ((0, 0), (5, k // 64 - 1), (70 % n, 1 % (k // 64)), (n - 1, 0)):
        w[r, 64 * grp: 64 * grp + 64] = rng.permutation(g)
    return w


def packed(w16, bits, group=64):
    codes, s16, z = oracle.quantize(w16, bits, group)
    n, k = w16.shape
    words = oracle.pack_codes(codes, bits).view(np.int32)
    qw = qlin.QWeight(n, k, bits, group, qlin.FMT_PACKED, dev(words),
                      dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
    return qw, oracle.dequantize(codes, s16, z, group)


def check(Y, X, what, label):
    assert np.all(np.isfinite(Y)), f"{label}: non-finite output"
    ref = oracle.matmul_ref(X, what)
    t = oracle.tolerance_scale(X, what)
    err = float(np.max(np.abs(Y.astype(np.float64) - ref)))
    assert err <= TOL * t, f"{label}: max err {err:.3e} > {TOL} * {t:.3e}"


# (form, splits, m): K-split 32 / 64 / 128 X rows (whole, pairs, halves),
# weights decoded once per work-group, the skinny kernel, the tiled kernels
FORMS = [(None, 1, 8), (None, 1, 100), (None, 1, 300), ("0,1", 1, 40), ("0,2", 2, 40),
         ("1,1", 1, 100), ("2,1", 1, 100), ("3,2", 2, 40), ("4,1", 1, 8), ("5,1", 1, 100),
         ("6,1", 1, 128), ("7,2", 2, 128), ("8,1", 1, 128), ("8,3", 3, 300), ("16,1", 1, 8),
         ("32,1", 1, 300), ("64,1", 1, 300), ("128,2", 2, 300)]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("where", ["bound", "beyond"])
@pytest.mark.parametrize("form,splits,m", FORMS)
def test_gemm_fp16_operand_range(bits, where, form, splits, m, launch_override):
    if form == "16,1" and bits in (5, 6, 7):
        pytest.skip("the skinny kernel exists for 2, 3, 4 and 8 bits")
    launch_override("gemm", form)
    L = ADMISSIBLE[bits] if where == "bound" else 65504
    n, k = 192, 640
    w16 = masters(bits, L, n, k, seed=bits * 7 + m)
    qw, what = packed(w16, bits)
    if where == "bound":
        assert np.all(np.isfinite(what.astype(np.float16)))
    else:
        with np.errstate(over="ignore"):
            assert not np.all(np.isfinite(what.astype(np.float16)))
    X = synth.activations(np.random.default_rng(m), m, k)
    print(f"gemm range bits={bits} {where} form={form} m={m}", flush=True)
    check(host(qlin.gemm(qw, dev(X))), X, what, f"{where} form={form} m={m}")
    # a two-matrix set: one ordinary matrix beside the extreme one
    w2 = synth.master_weights(np.random.default_rng(bits), 128, k)
    q2, what2 = packed(w2, bits)
    Y1, Y2 = qlin.gemm_multi([q2, qw], dev(X))
    check(host(Y1), X, what2, f"set[0] {where} form={form}")
    check(host(Y2), X, what, f"set[1] {where} form={form}")


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("form,m", [(None, 8), (None, 128), (None, 2048), ("1,1", 100),
                                    ("4,1", 40), ("7,1", 128), ("8,1", 128), ("8,2", 300),
                                    ("64,1", 300)])
def test_gemm_swiglu_fp16_operand_range(bits, form, m, launch_override):
    launch_override("gemm", form)
    n, k = 192, 640
    wg16 = masters(bits, 65504, n, k, seed=bits + 3)
    wu16 = synth.master_weights(np.random.default_rng(bits + 4), n, k)
    gate, wg = packed(wg16, bits)
    up, wu = packed(wu16, bits)
    X = synth.activations(np.random.default_rng(m + 1), m, k)
    print(f"gemm swiglu range bits={bits} form={form} m={m}", flush=True)
    H, _ = qlin.gemm_swiglu(gate, up, dev(X), want_h16=False)
    H = host(H)
    assert np.all(np.isfinite(H))
    ref = oracle.swiglu_ref(X, wg, wu)
    bound = oracle.swiglu_tolerance(X, wg, wu)
    assert np.all(np.abs(H.astype(np.float64) - ref) <= bound)


# The K-split kernel copies the scales of its K range to LDS and checks them
# after its K loop; a K range whose scales do not fit there is scanned before
# the loop instead.  These K reach that path: 4-wave work-groups over half
# tiles (k = 8256, 129 groups), over tile pairs (two tiles' scales), over
# whole tiles (k = 16448), and the 16-wave form at M <= 16 (k = 33280).
LONG_K = [("4,1", 40, 8256), ("3,1", 40, 8256), ("0,1", 40, 16448), ("4,1", 8, 33280)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("form,m,k", LONG_K)
def test_gemm_fp16_operand_range_long_k(bits, form, m, k, launch_override):
    launch_override("gemm", form)
    n = 192
    w16 = masters(bits, 65504, n, k, seed=bits * 11 + m)
    qw, what = packed(w16, bits)
    X = synth.activations(np.random.default_rng(m + k), m, k)
    print(f"gemm range long K bits={bits} form={form} m={m} k={k}", flush=True)
    check(host(qlin.gemm(qw, dev(X))), X, what, f"long K form={form} m={m} k={k}")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_gemm_swiglu_fp16_operand_range_long_k(bits, launch_override):
    """The pair over half tiles holds two tiles' scales: k = 4160 (65 groups)
    no longer fits, and the pair is scanned before its K loop."""
    launch_override("gemm", "4,1")
    n, k, m = 192, 4160, 40
    wg16 = masters(bits, 65504, n, k, seed=bits + 13)
    wu16 = synth.master_weights(np.random.default_rng(bits + 14), n, k)
    gate, wg = packed(wg16, bits)
    up, wu = packed(wu16, bits)
    X = synth.activations(np.random.default_rng(m + 7), m, k)
    print(f"gemm swiglu range long K bits={bits}", flush=True)
    H, _ = qlin.gemm_swiglu(gate, up, dev(X), want_h16=False)
    H = host(H)
    assert np.all(np.isfinite(H))
    ref = oracle.swiglu_ref(X, wg, wu)
    bound = oracle.swiglu_tolerance(X, wg, wu)
    assert np.all(np.abs(H.astype(np.float64) - ref) <= bound)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("form,m", [(None, 8), (None, 100), ("0,2", 40), ("3,1", 40),
                                    ("32,1", 300)])
def test_gemm_fp16_operand_range_per_channel(bits, form, m, launch_override):
    """Per-channel scales (one group per row, group = k): the extreme rows'
    single scale needs the operand scaling over the whole K range, in the
    K-split kernel (one work-group or two splits) and the tiled one."""
    launch_override("gemm", form)
    n, k = 192, 1280
    w16 = masters(bits, 65504, n, k, seed=bits * 5 + m)
    qw, what = packed(w16, bits, group=k)
    with np.errstate(over="ignore"):
        assert not np.all(np.isfinite(what.astype(np.float16)))
    X = synth.activations(np.random.default_rng(m + 3), m, k)
    print(f"gemm range per-channel bits={bits} form={form} m={m}", flush=True)
    check(host(qlin.gemm(qw, dev(X))), X, what, f"per-channel form={form} m={m}")
