"""GPU parity of qlin_gemm_swiglu (the prefill gate/up GEMM with the SwiGLU
combination) against the CPU oracle.

* H within the bound the GEMM tolerance implies for silu(g) * u at every
  output (oracle.swiglu_tolerance with X of m rows), H16 = fp16(H) nearest
  even, bit for bit, and within that bound plus fp16 rounding of the oracle.
* One-hot X rows: g and u are then single dequantized weights rounded to fp16
  (the GEMM's operand rounding), so H must equal silu(g) * u of those fp16
  values to within the fp32 evaluation of silu and the product.
* Every kernel form (K-split with 32 / 64 X rows, also over half tiles, LDS
  pipeline with 64 / 128 X rows, with and without a K split across
  work-groups), ragged n (an odd
  tile count leaves half of the last pair's work-group without a tile) and
  ragged m; reruns bitwise identical; either output alone gives the same
  values.
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


def check_swiglu(H, H16, X, wg, wu, label):
    ref = oracle.swiglu_ref(X, wg, wu)
    bound = oracle.swiglu_tolerance(X, wg, wu)
    if H is not None:
        err = np.abs(H.astype(np.float64) - ref)
        i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        assert np.all(err <= bound), f"{label}: H{i} err {err[i]:.3e} > bound {bound[i]:.3e}"
    if H16 is not None:
        err16 = np.abs(H16.astype(np.float64) - ref)
        b16 = bound + np.abs(ref) * 2.0 ** -11 + 2.0 ** -25
        assert np.all(err16 <= b16), f"{label}: H16 outside bound"
    if H is not None and H16 is not None:
        assert np.array_equal(H.astype(np.float16).view(np.uint16), H16.view(np.uint16))


def check_one_hot(gate, up, wg, wu, k, label, rng):
    """X rows one-hot at columns cs: H[i] = silu(fp16(wg[:, c_i])) * fp16(wu[:, c_i])."""
    cs = np.unique(np.concatenate([[0, k - 1], rng.integers(0, k, 6)]))
    X = np.zeros((len(cs), k), np.float16)
    X[np.arange(len(cs)), cs] = 1
    H, H16 = qlin.gemm_swiglu(gate, up, dev(X))
    g = wg[:, cs].T.astype(np.float32).astype(np.float16).astype(np.float64)
    u = wu[:, cs].T.astype(np.float32).astype(np.float16).astype(np.float64)
    ref = oracle.silu(g) * u
    err = np.abs(host(H).astype(np.float64) - ref)
    assert np.all(err <= 4e-6 * np.abs(ref) + 1e-30), f"{label}: one-hot max err {err.max():.3e}"
    assert np.array_equal(host(H).astype(np.float16).view(np.uint16), host(H16).view(np.uint16))


# (n, k, m): the kernel forms the default policy picks, small M to 2048
DEFAULT_CASES = [
    (200, 192, 1),        # K-split, 32 X rows, K split across work-groups
    (200, 192, 17),
    (130, 640, 100),      # three tiles (odd)
    (896, 896, 128),
    (4864, 896, 40),      # many tiles, M <= 256
    (640, 8192, 40),      # long K: split across work-groups
    (896, 896, 300),      # M > 256, few columns: K-split with 64 X rows
]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
@pytest.mark.parametrize("n,k,m", DEFAULT_CASES)
def test_gemm_swiglu(bits, group, n, k, m, launch_override):
    launch_override("gemm", None)
    g = k if group == "K" else group
    rng = np.random.default_rng([81, bits, n, k, m])
    gate, wg = packed(synth.master_weights(rng, n, k), bits, g)
    up, wu = packed(synth.master_weights(rng, n, k), bits, g)
    X = synth.activations(rng, m, k)
    say(f"gemm_swiglu bits={bits} group={g} n={n} k={k} m={m}")
    Xd = dev(X)
    H, H16 = qlin.gemm_swiglu(gate, up, Xd)
    hh, hh16 = host(H), host(H16)
    check_swiglu(hh, hh16, X, wg, wu, f"{n}x{k} m={m}")
    H2, H162 = qlin.gemm_swiglu(gate, up, Xd)
    assert np.array_equal(hh, host(H2)) and np.array_equal(hh16, host(H162))
    only32, none16 = qlin.gemm_swiglu(gate, up, Xd, want_h16=False)
    assert none16 is None and np.array_equal(host(only32), hh)
    none32, only16 = qlin.gemm_swiglu(gate, up, Xd, want_h=False)
    assert none32 is None and np.array_equal(host(only16), hh16)


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_gemm_swiglu_prefill_m2048(bits, launch_override):
    """The Qwen2.5-0.5B gate/up shape at M = 2048: the LDS pipeline with
    128-row X tiles; sampled rows checked against the oracle."""
    launch_override("gemm", None)
    n, k, m = 4864, 896, 2048
    rng = np.random.default_rng([82, bits])
    gate, wg = packed(synth.master_weights(rng, n, k), bits, 64)
    up, wu = packed(synth.master_weights(rng, n, k), bits, 64)
    X = synth.activations(rng, m, k)
    say(f"gemm_swiglu m2048 bits={bits}")
    H, H16 = qlin.gemm_swiglu(gate, up, dev(X))
    rows = np.unique(np.concatenate([[0, 127, 128, m - 1], rng.integers(0, m, 12)]))
    hh, hh16 = host(H)[rows], host(H16)[rows]
    # the tolerance scale is the whole product's: max over all rows of sum |x w|
    T = oracle.tolerance_scale(X, wg), oracle.tolerance_scale(X, wu)
    g = oracle.matmul_ref(X[rows], wg)
    u = oracle.matmul_ref(X[rows], wu)
    ref = oracle.silu(g) * u
    eg, eu = 1e-3 * T[0], 1e-3 * T[1]
    bound = (oracle.SILU_SLOPE_MAX * eg * (np.abs(u) + eu) + np.abs(oracle.silu(g)) * eu
             + 4e-6 * np.abs(ref))
    err = np.abs(hh.astype(np.float64) - ref)
    assert np.all(err <= bound), f"max err {err.max():.3e}"
    assert np.array_equal(hh.astype(np.float16).view(np.uint16), hh16.view(np.uint16))


# "mb,splits": K-split with 32 (0) / 64 (1) X rows, the same over half tiles
# (4 / 5), the form decoding each weight once per work-group (8), LDS
# pipeline with 64 / 128 X rows (32 runs as 64), with and without a K split
# across work-groups
FORCED = ["0,1", "0,3", "1,1", "1,2", "4,1", "4,3", "5,1", "5,2", "6,1", "7,2", "8,1", "8,2",
          "32,1", "64,1", "64,2", "128,1", "128,3"]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("cfg", FORCED)
@pytest.mark.parametrize("n,k,m", [(130, 640, 150), (256, 192, 70), (64, 1024, 3)])
def test_gemm_swiglu_forms(bits, cfg, n, k, m, launch_override):
    launch_override("gemm", cfg)
    rng = np.random.default_rng([83, bits, n, k, m])
    gate, wg = packed(synth.master_weights(rng, n, k), bits, 64)
    up, wu = packed(synth.master_weights(rng, n, k), bits, 64)
    X = synth.activations(rng, m, k)
    say(f"gemm_swiglu cfg={cfg} bits={bits} n={n} k={k} m={m}")
    Xd = dev(X)
    H, H16 = qlin.gemm_swiglu(gate, up, Xd)
    hh, hh16 = host(H), host(H16)
    check_swiglu(hh, hh16, X, wg, wu, f"{cfg} {n}x{k} m={m}")
    H2, _ = qlin.gemm_swiglu(gate, up, Xd)
    assert np.array_equal(hh, host(H2))
    check_one_hot(gate, up, wg, wu, k, cfg, rng)


def test_gemm_swiglu_strided_outputs(launch_override):
    """H and H16 with a row stride above n (ld_h = n + 24): the padding is
    left untouched, the rows hold what the packed call gives."""
    launch_override("gemm", None)
    n, k, m = 200, 192, 300
    rng = np.random.default_rng(84)
    gate, wg = packed(synth.master_weights(rng, n, k), 4, 64)
    up, wu = packed(synth.master_weights(rng, n, k), 4, 64)
    Xd = dev(synth.activations(rng, m, k))
    say("gemm_swiglu strided outputs")
    Hp = torch.full((m, n + 24), 7.0, dtype=torch.float32, device=DEV)
    H16p = torch.full((m, n + 24), 3.0, dtype=torch.float16, device=DEV)
    qlin.gemm_swiglu(gate, up, Xd, Hp[:, :n], H16p[:, :n])
    H, H16 = qlin.gemm_swiglu(gate, up, Xd)
    hp, h16p = host(Hp), host(H16p)
    assert np.array_equal(hp[:, :n], host(H)) and np.array_equal(h16p[:, :n], host(H16))
    assert np.all(hp[:, n:] == 7.0) and np.all(h16p[:, n:] == 3.0)


def test_gemm_swiglu_extremes(launch_override):
    """Large |g|: silu saturates to g (g >> 0) and to -0 (g << 0) without nan."""
    launch_override("gemm", None)
    rng = np.random.default_rng(85)
    n, k, m = 256, 256, 40
    gate, wg = packed(synth.master_weights(rng, n, k) * np.float16(40), 8, 64)
    up, wu = packed(synth.master_weights(rng, n, k), 8, 64)
    X = synth.activations(rng, m, k)
    say("gemm_swiglu extremes")
    H, H16 = qlin.gemm_swiglu(gate, up, dev(X))
    hh = host(H)
    assert not np.any(np.isnan(hh))
    check_swiglu(hh, host(H16), X, wg, wu, "extremes")
