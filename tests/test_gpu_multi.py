"""GPU parity of the multi-matrix decode launches against the CPU oracle.

* qlin_gemv_multi: each y_i within max |y - y_ref| <= 1e-3 * max_row sum |x w|
  of its own matrix (the single-GEMV bound), with one-hot x exact; sets of
  1..4 matrices with ragged n, with and without split-K.
* qlin_gemv_swiglu: h within the bound the GEMV tolerance implies for
  silu(g) * u (oracle.swiglu_tolerance), h16 = fp16(h) nearest even, bit for
  bit, and within that bound plus fp16 rounding of the oracle's h.
* Both are deterministic (bitwise identical reruns).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from group_wise_bit_amd import qlin

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def packed(w16, bits, group):
    codes, s16, z = oracle.quantize(w16, bits, group)
    n, k = w16.shape
    words = oracle.pack_codes(codes, bits).view(np.int32)
    qw = qlin.QWeight(n, k, bits, group, qlin.FMT_PACKED, dev(words),
                      dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
    return qw, oracle.dequantize(codes, s16, z, group)


def check_tol(y, x16, what, label):
    ref = oracle.matmul_ref(x16, what)
    t = oracle.tolerance_scale(x16, what)
    err = float(np.max(np.abs(y.astype(np.float64) - ref)))
    assert err <= 1e-3 * t, f"{label}: max err {err:.3e} > 1e-3 * {t:.3e}"


MULTI_CASES = [
    ((896, 128, 128), 896),          # Qwen2.5-0.5B q, k, v
    ((200, 64, 1, 130), 192),        # ragged rows, four matrices
    ((2048, 1024, 1024), 1024),      # Qwen3-0.6B q, k, v
    ((4096, 1024, 1024), 4096),      # Qwen3-8B q, k, v
    ((77,), 640),                    # a set of one
]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
@pytest.mark.parametrize("ns,k", MULTI_CASES)
def test_gemv_multi(bits, group, ns, k):
    g = k if group == "K" else group
    rng = np.random.default_rng([71, bits, k, len(ns)])
    mats = [packed(synth.master_weights(rng, n, k), bits, g) for n in ns]
    x16 = synth.activations(rng, 1, k)[0]
    say(f"gemv_multi bits={bits} group={g} ns={ns} k={k}")
    xd = dev(x16)
    ys = qlin.gemv_multi([m[0] for m in mats], xd)
    out = [host(y) for y in ys]
    for i, (y, (_, what)) in enumerate(zip(out, mats)):
        check_tol(y, x16, what, f"matrix {i}")
    again = [host(y) for y in qlin.gemv_multi([m[0] for m in mats], xd)]
    for a, b in zip(out, again):
        assert np.array_equal(a, b)
    # one-hot x: y_i = column c of the dequantized weights, exactly
    c = int(rng.integers(0, k))
    e = np.zeros(k, dtype=np.float16); e[c] = 1
    for y, (_, what) in zip(qlin.gemv_multi([m[0] for m in mats], dev(e)), mats):
        assert np.array_equal(host(y).astype(np.float64), what[:, c])


def test_gemv_multi_shared_workspace_counters():
    rng = np.random.default_rng(72)
    k = 8192
    mats = [packed(synth.master_weights(rng, n, k), 4, 64) for n in (640, 128)]
    x16 = synth.activations(rng, 1, k)[0]
    need = qlin.library().qlin_gemv_multi_workspace_bytes(
        (qlin.QlinWeightC * 2)(*[m[0].c_struct() for m in mats]), 2)
    assert need > 65536
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    say("gemv_multi split-K with explicit workspace")
    ys = [host(y) for y in qlin.gemv_multi([m[0] for m in mats], dev(x16), ws=ws)]
    for y, (_, what) in zip(ys, mats):
        check_tol(y, x16, what, "split")
    assert torch.count_nonzero(ws[:65536]).item() == 0
    ws[65536:].fill_(0x7F)
    ys2 = [host(y) for y in qlin.gemv_multi([m[0] for m in mats], dev(x16), ws=ws)]
    for a, b in zip(ys, ys2):
        assert np.array_equal(a, b)


SWIGLU_CASES = [(4864, 896), (3072, 1024), (12288, 4096), (1024, 4096), (130, 192), (1, 64)]


def check_swiglu(h, h16, x16, wg, wu, label):
    ref = oracle.swiglu_ref(x16, wg, wu)
    bound = oracle.swiglu_tolerance(x16, wg, wu)
    if h is not None:
        err = np.abs(h.astype(np.float64) - ref)
        i = int(np.argmax(err - bound))
        assert np.all(err <= bound), f"{label}: h[{i}] err {err[i]:.3e} > bound {bound[i]:.3e}"
    if h16 is not None:
        err16 = np.abs(h16.astype(np.float64) - ref)
        b16 = bound + np.abs(ref) * 2.0 ** -11 + 2.0 ** -25
        assert np.all(err16 <= b16), f"{label}: h16 outside bound"
    if h is not None and h16 is not None:
        assert np.array_equal(h.astype(np.float16).view(np.uint16), h16.view(np.uint16))


# launch shapes "waves,splits,rows per work-group" (whole tiles, 16 / 8 rows)
ROW_WIDTHS = ["16,1,64", "8,1,16", "16,1,8", "4,3,8", "8,2,16", "8,3,64"]


@pytest.mark.parametrize("bits", [3, 4, 6])
@pytest.mark.parametrize("cfg", ROW_WIDTHS)
@pytest.mark.parametrize("ns,k", [((200, 64, 1, 130), 192), ((896, 128, 128), 896)])
def test_gemv_multi_row_widths(bits, cfg, ns, k, launch_override):
    """Sets of matrices at every work-group width: each output within its
    matrix's tolerance; one-hot x exact."""
    launch_override("gemv", cfg)
    rng = np.random.default_rng([75, bits, k, len(ns)])
    mats = [packed(synth.master_weights(rng, n, k), bits, 64) for n in ns]
    x16 = synth.activations(rng, 1, k)[0]
    say(f"gemv_multi cfg={cfg} bits={bits} ns={ns} k={k}")
    for i, (y, (_, what)) in enumerate(zip(qlin.gemv_multi([m[0] for m in mats], dev(x16)), mats)):
        check_tol(host(y), x16, what, f"{cfg} matrix {i}")
    for c in (0, 37, k - 1):
        e = np.zeros(k, dtype=np.float16); e[c] = 1
        for y, (_, what) in zip(qlin.gemv_multi([m[0] for m in mats], dev(e)), mats):
            assert np.array_equal(host(y).astype(np.float64), what[:, c]), f"{cfg} one-hot {c}"


@pytest.mark.parametrize("bits", [3, 4, 6])
@pytest.mark.parametrize("cfg", ROW_WIDTHS)
@pytest.mark.parametrize("n,k", [(130, 192), (200, 1024)])
def test_gemv_swiglu_row_widths(bits, cfg, n, k, launch_override):
    launch_override("gemv", cfg)
    rng = np.random.default_rng([76, bits, n, k])
    gate, wg = packed(synth.master_weights(rng, n, k), bits, 64)
    up, wu = packed(synth.master_weights(rng, n, k), bits, 64)
    x16 = synth.activations(rng, 1, k)[0]
    say(f"gemv_swiglu cfg={cfg} bits={bits} n={n} k={k}")
    h, h16 = qlin.gemv_swiglu(gate, up, dev(x16))
    check_swiglu(host(h), host(h16), x16, wg, wu, f"{cfg} swiglu {n}x{k}")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
@pytest.mark.parametrize("n,k", SWIGLU_CASES)
def test_gemv_swiglu(bits, group, n, k):
    g = k if group == "K" else group
    rng = np.random.default_rng([73, bits, n, k])
    gate, wg = packed(synth.master_weights(rng, n, k), bits, g)
    up, wu = packed(synth.master_weights(rng, n, k), bits, g)
    x16 = synth.activations(rng, 1, k)[0]
    say(f"gemv_swiglu bits={bits} group={g} n={n} k={k}")
    xd = dev(x16)
    h, h16 = qlin.gemv_swiglu(gate, up, xd)
    hh, hh16 = host(h), host(h16)
    check_swiglu(hh, hh16, x16, wg, wu, f"swiglu {n}x{k}")
    h2, h162 = qlin.gemv_swiglu(gate, up, xd)
    assert np.array_equal(hh, host(h2)) and np.array_equal(hh16, host(h162))
    # either output alone gives the same values
    only32, none16 = qlin.gemv_swiglu(gate, up, xd, want_h16=False)
    assert none16 is None and np.array_equal(host(only32), hh)
    none32, only16 = qlin.gemv_swiglu(gate, up, xd, want_h=False)
    assert none32 is None and np.array_equal(host(only16), hh16)


def test_gemv_swiglu_extremes():
    """Large |g|: silu saturates to g (g >> 0) and to -0 (g << 0) without nan."""
    rng = np.random.default_rng(74)
    n, k = 256, 256
    w = synth.master_weights(rng, n, k) * np.float16(40)       # |g| up to ~100
    gate, wg = packed(w, 8, 64)
    up, wu = packed(synth.master_weights(rng, n, k), 8, 64)
    x16 = synth.activations(rng, 1, k)[0]
    say("gemv_swiglu extremes")
    h, h16 = qlin.gemv_swiglu(gate, up, dev(x16))
    hh, hh16 = host(h), host(h16)
    assert not np.any(np.isnan(hh))
    check_swiglu(hh, hh16, x16, wg, wu, "extremes")


GEMM_MULTI_CASES = [
    ((896, 128, 128), 896, 8),       # skinny (M <= 16)
    ((896, 128, 128), 896, 17),
    ((896, 128, 128), 896, 128),
    ((200, 64, 1, 130), 192, 100),   # four ragged matrices
    ((4864, 4864), 896, 2048),       # gate/up at M = 2048: 128-row tiles
    ((896, 128, 128), 896, 300),
    ((640, 128), 8192, 100),         # split K
    ((2048, 1024, 1024), 1024, 1),
]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("ns,k,m", GEMM_MULTI_CASES)
def test_gemm_multi(bits, ns, k, m):
    rng = np.random.default_rng([75, bits, k, m, len(ns)])
    mats = [packed(synth.master_weights(rng, n, k), bits, 64) for n in ns]
    X = synth.activations(rng, m, k)
    say(f"gemm_multi bits={bits} ns={ns} k={k} m={m}")
    Xd = dev(X)
    Ys = [host(y) for y in qlin.gemm_multi([q for q, _ in mats], Xd)]
    for i, (Y, (_, what)) in enumerate(zip(Ys, mats)):
        check_tol(Y, X, what, f"matrix {i}")
    again = [host(y) for y in qlin.gemm_multi([q for q, _ in mats], Xd)]
    for a, b in zip(Ys, again):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("cfg", ["0,1", "3,1", "4,2", "16,1", "32,1", "64,1", "128,1"])
@pytest.mark.parametrize("m", [8, 100])
def test_gemm_multi_forced_forms(bits, cfg, m, launch_override):
    """A ragged three-matrix set through every GEMM kernel form forced by
    the launch-shape override, also the tiled kernels at M <= 16 (their
    launch columns are four-tile columns, not the K-split kernel's tiles):
    every matrix's Y within tolerance."""
    launch_override("gemm", cfg)
    rng = np.random.default_rng([76, bits, m])
    k = 640
    mats = [packed(synth.master_weights(rng, n, k), bits, 64) for n in (200, 64, 130)]
    X = synth.activations(rng, m, k)
    say(f"gemm_multi forced cfg={cfg} bits={bits} m={m}")
    Ys = [host(y) for y in qlin.gemm_multi([q for q, _ in mats], dev(X))]
    for i, (Y, (_, what)) in enumerate(zip(Ys, mats)):
        check_tol(Y, X, what, f"{cfg} matrix {i}")
