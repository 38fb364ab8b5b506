"""GPU parity of the GEMM form that decodes each weight once per work-group
(k_gemm_wdec: 128 X rows x a tile pair, or x tile t of gate and of up) against
the CPU oracle, reached through the launch-shape override (form 8).

* qlin_gemm / qlin_gemm_multi: every Y within max |y - y_ref| <= 1e-3 *
  max_row sum |x w| (the GEMM bound), one-hot X rows exact (the dequantized
  weight rounded to fp16, the operand's rounding); odd tile counts (the last
  work-group's second tile re-read and not stored), ragged n and m, K ranges
  that leave 0-3 blocks after the last full round of four, per-channel
  scales, K split across work-groups (1, 2, 3 ways), widths 2-8; reruns
  bitwise identical.
* qlin_gemm_swiglu: H within the bound the GEMM tolerance implies for
  silu(g) * u, H16 = fp16(H) bit for bit.
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
    words = oracle.pack_codes(codes, bits).view(np.int32)
    n, k = w16.shape
    qw = qlin.QWeight(n, k, bits, group, qlin.FMT_PACKED, dev(words),
                      dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
    return qw, oracle.dequantize(codes, s16, z, group)


def check_tol(Y, X, what, label):
    assert np.all(np.isfinite(Y)), f"{label}: non-finite output"
    ref = oracle.matmul_ref(X, what)
    t = oracle.tolerance_scale(X, what)
    err = float(np.max(np.abs(Y.astype(np.float64) - ref)))
    assert err <= 1e-3 * t, f"{label}: max err {err:.3e} > 1e-3 * {t:.3e}"


def check_one_hot(qw, what, k, label, rng):
    """X rows one-hot at columns cs: Y[i] = fp16(what[:, c_i]) exactly."""
    cs = np.unique(np.concatenate([[0, k - 1], rng.integers(0, k, 6)]))
    X = np.zeros((len(cs), k), np.float16)
    X[np.arange(len(cs)), cs] = 1
    Y = host(qlin.gemm(qw, dev(X)))
    ref = what[:, cs].T.astype(np.float32).astype(np.float16).astype(np.float32)
    assert np.array_equal(Y, ref), f"{label}: one-hot differs"


# (n, k, m): odd and even tile counts, ragged n and m, K-block counts 10
# (4 + 4 + 2), 3 (no full round), 13 (4 * 3 + 1), 64
CASES = [(130, 640, 100), (200, 192, 128), (64, 832, 257), (300, 4096, 40), (1000, 640, 1)]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("splits", [1, 2, 3])
@pytest.mark.parametrize("n,k,m", CASES)
def test_gemm_wdec(bits, splits, n, k, m, launch_override):
    launch_override("gemm", f"8,{splits}")
    rng = np.random.default_rng([91, bits, n, k, m, splits])
    qw, what = packed(synth.master_weights(rng, n, k), bits, 64)
    X = synth.activations(rng, m, k)
    say(f"gemm wdec bits={bits} splits={splits} n={n} k={k} m={m}")
    Xd = dev(X)
    Y = host(qlin.gemm(qw, Xd))
    check_tol(Y, X, what, f"{n}x{k} m={m} splits={splits}")
    assert np.array_equal(Y, host(qlin.gemm(qw, Xd)))
    check_one_hot(qw, what, k, f"{n}x{k} splits={splits}", rng)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("splits", [1, 2])
def test_gemm_wdec_per_channel(bits, splits, launch_override):
    launch_override("gemm", f"8,{splits}")
    n, k, m = 192, 704, 150
    rng = np.random.default_rng([92, bits, splits])
    qw, what = packed(synth.master_weights(rng, n, k), bits, k)
    X = synth.activations(rng, m, k)
    say(f"gemm wdec per-channel bits={bits} splits={splits}")
    check_tol(host(qlin.gemm(qw, dev(X))), X, what, "per-channel")
    check_one_hot(qw, what, k, "per-channel", rng)


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("cfg", ["8,1", "8,2"])
@pytest.mark.parametrize("m", [8, 100, 300])
def test_gemm_multi_wdec(bits, cfg, m, launch_override):
    """A ragged set whose matrices all have even tile counts (tile pairs stay
    within one matrix), and one that has not (the launch falls back to
    another form): every Y within tolerance."""
    launch_override("gemm", cfg)
    rng = np.random.default_rng([93, bits, m])
    k = 640
    for ns in ((200, 128, 250), (200, 64, 130)):
        mats = [packed(synth.master_weights(rng, n, k), bits, 64) for n in ns]
        X = synth.activations(rng, m, k)
        say(f"gemm_multi wdec cfg={cfg} bits={bits} m={m} ns={ns}")
        Ys = [host(y) for y in qlin.gemm_multi([q for q, _ in mats], dev(X))]
        for i, (Y, (_, what)) in enumerate(zip(Ys, mats)):
            check_tol(Y, X, what, f"{cfg} {ns} matrix {i}")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("n,k,m", [(130, 640, 150), (256, 192, 70), (64, 1024, 3)])
def test_gemm_swiglu_wdec(bits, splits, n, k, m, launch_override):
    launch_override("gemm", f"8,{splits}")
    rng = np.random.default_rng([94, bits, n, k, m, splits])
    gate, wg = packed(synth.master_weights(rng, n, k), bits, 64)
    up, wu = packed(synth.master_weights(rng, n, k), bits, 64)
    X = synth.activations(rng, m, k)
    say(f"gemm_swiglu wdec bits={bits} splits={splits} n={n} k={k} m={m}")
    Xd = dev(X)
    H, H16 = qlin.gemm_swiglu(gate, up, Xd)
    hh, hh16 = host(H), host(H16)
    ref = oracle.swiglu_ref(X, wg, wu)
    bound = oracle.swiglu_tolerance(X, wg, wu)
    err = np.abs(hh.astype(np.float64) - ref)
    assert np.all(err <= bound), f"max err {err.max():.3e}"
    assert np.array_equal(hh.astype(np.float16).view(np.uint16), hh16.view(np.uint16))
    H2, _ = qlin.gemm_swiglu(gate, up, Xd)
    assert np.array_equal(hh, host(H2))


@pytest.mark.parametrize("bits", [4, 3])
def test_gemm_wdec_qwen3_8b_m128(bits, launch_override):
    """The Qwen3-8B gate/up pair (12288 x 4096) at M = 128 through this form:
    sampled output columns against the oracle (the tolerance scale of the
    sampled columns' weights)."""
    launch_override("gemm", "8,1")
    n, k, m = 12288, 4096, 128
    rng = np.random.default_rng([95, bits])
    cols = np.unique(np.concatenate([[0, 63, 64, 127, n - 1], rng.integers(0, n, 40)]))
    wg16 = synth.master_weights(rng, n, k)
    wu16 = synth.master_weights(rng, n, k)
    gate, _ = packed(wg16, bits, 64)
    up, _ = packed(wu16, bits, 64)
    X = synth.activations(rng, m, k)
    say(f"gemm_swiglu wdec qwen3-8b m128 bits={bits}")
    H, _ = qlin.gemm_swiglu(gate, up, dev(X), want_h16=False)
    hh = host(H)[:, cols]
    cg, sg, zg = oracle.quantize(wg16[cols], bits, 64)
    cu, su, zu = oracle.quantize(wu16[cols], bits, 64)
    wg = oracle.dequantize(cg, sg, zg, 64)
    wu = oracle.dequantize(cu, su, zu, 64)
    ref = oracle.swiglu_ref(X, wg, wu)
    bound = oracle.swiglu_tolerance(X, wg, wu)
    err = np.abs(hh.astype(np.float64) - ref)
    assert np.all(err <= bound), f"max err {err.max():.3e}"
