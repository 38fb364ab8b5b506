"""GPU parity: the HIP path through the C ABI against the CPU oracle.

* qlin_quantize: packed words, codes, fp16 scales and zeros bit-exact.
* qlin_gemv / qlin_gemm: max |y - y_ref| <= 1e-3 * max_row sum_k |x_k w_k|
  (y_ref in binary64 from the oracle's dequantized weights), and, with
  one-hot inputs, the output equals a column of the dequantized weights
  exactly (GEMV: the fp32 value s*(q - z); GEMM: that value rounded to fp16),
  which checks every decoded / re-rounded code bit for bit.
* Deterministic: two runs give bitwise identical outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from group_wise_bit_amd import qlin

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-3


def say(msg):
    print(msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def oracle_packed(w16, bits, group):
    codes, s16, z = oracle.quantize(w16, bits, group)
    n, k = w16.shape
    words = oracle.pack_codes(codes, bits).view(np.int32)
    qw = qlin.QWeight(n, k, bits, group, qlin.FMT_PACKED, dev(words),
                      dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
    return qw, codes, s16, z


def check_tol(y, x16, what, label):
    ref = oracle.matmul_ref(x16, what)
    t = oracle.tolerance_scale(x16, what)
    err = float(np.max(np.abs(y.astype(np.float64) - ref))) if ref.size else 0.0
    assert err <= TOL * t, f"{label}: max err {err:.3e} > {TOL} * {t:.3e}"
    return err / (TOL * t) if t > 0 else 0.0


def fp16_rne(a64):
    """binary64 values that are exact in binary32 -> fp16 (nearest even), as float64."""
    return np.asarray(a64, dtype=np.float32).astype(np.float16).astype(np.float64)


SHAPES = [(896, 896), (200, 192), (64, 64), (1, 64), (130, 256)]


# ------------------------------------------------------------- quantize --
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
@pytest.mark.parametrize("shape", SHAPES + [(2048, 1024)])
def test_quantize_bit_exact(bits, group, shape):
    n, k = shape
    g = k if group == "K" else 64
    say(f"quantize bits={bits} group={g} shape={shape}")
    rng = np.random.default_rng(n * 31 + k + bits)
    w16 = synth.master_weights(rng, n, k)
    codes, s16, z = oracle.quantize(w16, bits, g)
    qw = qlin.quantize(dev(w16), bits, g)
    words = host(qw.data).view(np.uint32)
    assert np.array_equal(words, oracle.pack_codes(codes, bits))
    assert np.array_equal(host(qw.scale).view(np.uint16), oracle.tile_meta(s16).view(np.uint16))
    assert np.array_equal(host(qw.zero), oracle.tile_meta(z))
    only = qlin.quantize(dev(w16), bits, g, codes=False)
    assert np.array_equal(host(only.scale).view(np.uint16), oracle.tile_meta(s16).view(np.uint16))
    assert np.array_equal(host(only.zero), oracle.tile_meta(z))


@pytest.mark.parametrize("bits", [5, 6, 7])
@pytest.mark.parametrize("group", [64, "K"])
def test_quantize_scale_zero_lever_widths(bits, group):
    """5-7 bits, scale and zero only (the fused path's precompute): bit-exact,
    also batched, on random and edge-case groups; the packed codes of the
    same call bit-exact too."""
    rng = np.random.default_rng(700 + bits)
    w16 = np.concatenate([synth.master_weights(rng, 130, 448),
                          synth.edge_groups(bits, rng, n_rows=64, k=448)])
    g = 448 if group == "K" else 64
    say(f"quantize scale/zero bits={bits} group={g}")
    q = qlin.quantize(dev(w16), bits, group, codes=False)
    qb = qlin.quantize_batch([dev(w16)], bits, group, codes=False)[0]
    s16, z = oracle.rtn_scale_zero(w16, bits, g)
    for got in (q, qb):
        assert np.array_equal(host(got.scale).view(np.uint16)[:oracle.tile_meta(s16).size],
                              oracle.tile_meta(s16).view(np.uint16))
        assert np.array_equal(host(got.zero)[:oracle.tile_meta(z).size], oracle.tile_meta(z))
    packed = qlin.quantize(dev(w16), bits, group, codes=True)
    codes = oracle.quantize(w16, bits, g)[0]
    assert np.array_equal(host(packed.data).view(np.uint32), oracle.pack_codes(codes, bits))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
def test_quantize_edge_groups(bits, group):
    rng = np.random.default_rng(77 + bits)
    w16 = synth.edge_groups(bits, rng, n_rows=96, k=512)
    g = 512 if group == "K" else 64
    say(f"quantize edge groups bits={bits} group={g}")
    codes, s16, z = oracle.quantize(w16, bits, g)
    qw = qlin.quantize(dev(w16), bits, g)
    got = oracle.unpack_codes(host(qw.data).view(np.uint32), 96, 512, bits)
    assert np.array_equal(got, codes)
    assert np.array_equal(host(qw.scale).view(np.uint16), oracle.tile_meta(s16).view(np.uint16))
    assert np.array_equal(host(qw.zero), oracle.tile_meta(z))


def test_quantize_worked_example_and_pitch():
    """Example A of tests/golden in row 3 of a strided matrix."""
    w = np.zeros((5, 200), np.float16)
    w[3, 64:128] = np.array([-1, 2, 0, 0.5, 1, -0.5] + [0] * 58, np.float16)
    full = dev(w)
    view = full[:, :128]                        # pitch 200 elements, k = 128
    qw = qlin.quantize(view, 4, 64)
    s = host(qw.scale).view(np.uint16)
    assert s[1 * 64 + 3] == 0x3266
    assert host(qw.zero)[1 * 64 + 3] == 5
    c = oracle.unpack_codes(host(qw.data).view(np.uint32), 5, 128, 4)
    assert list(c[3, 64:70]) == [0, 15, 5, 8, 10, 2]


# ------------------------------------------------------------------ GEMV --
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
@pytest.mark.parametrize("shape", SHAPES + [(1024, 4096), (128, 896)])
def test_gemv_packed(bits, group, shape):
    n, k = shape
    g = k if group == "K" else 64
    say(f"gemv packed bits={bits} group={g} shape={shape}")
    rng = np.random.default_rng(n + 7 * k + bits)
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, 1, k)[0]
    qw, codes, s16, z = oracle_packed(w16, bits, g)
    what = oracle.dequantize(codes, s16, z, g)
    y = host(qlin.gemv(qw, dev(x16)))
    check_tol(y, x16, what, "gemv")
    for kk in sorted({0, k // 2 + 3, k - 1}):
        e = np.zeros(k, np.float16)
        e[kk] = 1
        ye = host(qlin.gemv(qw, dev(e)))
        assert np.array_equal(ye.astype(np.float64), what[:, kk]), f"one-hot k={kk}"


# launch shapes "waves,splits,rows per work-group": whole 64-row tiles, and
# 16 / 8 rows over 4 / 8 slices of every block, with and without a K split
ROW_WIDTHS = ["16,1,64", "8,1,16", "16,1,8", "4,3,8", "8,2,16"]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
@pytest.mark.parametrize("shape", [(200, 192), (130, 4096), (1, 64), (896, 896)])
@pytest.mark.parametrize("cfg", ROW_WIDTHS)
def test_gemv_row_widths(bits, group, shape, cfg, launch_override):
    """Every work-group width of the packed GEMV: within tolerance, and one-hot
    x at positions covering every slice of the first and last block reproduces
    the dequantized column exactly."""
    launch_override("gemv", cfg)
    n, k = shape
    g = k if group == "K" else 64
    say(f"gemv packed cfg={cfg} bits={bits} group={g} shape={shape}")
    rng = np.random.default_rng([n, k, bits, 5])
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, 1, k)[0]
    qw, codes, s16, z = oracle_packed(w16, bits, g)
    what = oracle.dequantize(codes, s16, z, g)
    check_tol(host(qlin.gemv(qw, dev(x16))), x16, what, cfg)
    for kk in sorted(set(range(0, 64, 7)) | set(range(k - 64, k, 9))):
        e = np.zeros(k, np.float16)
        e[kk] = 1
        ye = host(qlin.gemv(qw, dev(e)))
        assert np.array_equal(ye.astype(np.float64), what[:, kk]), f"{cfg} one-hot k={kk}"


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
@pytest.mark.parametrize("shape", [(200, 4864), (70, 8192), (896, 4864)])
@pytest.mark.parametrize("cfg", [None, "16,1,8", "16,1,16"])
def test_gemv_narrow_long_k(bits, group, shape, cfg, launch_override):
    """16-wave 8- and 16-row work-groups over 65..128 K-blocks, where each wave
    takes two rounds of loads (the Qwen2.5-0.5B down projection, k = 4864,
    takes this form by default): within tolerance, and one-hot x in the first
    and last blocks gives the dequantized column exactly."""
    if cfg is None:
        launch_override("gemv", None)
    else:
        launch_override("gemv", cfg)
    n, k = shape
    g = k if group == "K" else 64
    say(f"gemv narrow long-k cfg={cfg} bits={bits} group={g} shape={shape}")
    rng = np.random.default_rng([n, k, bits, 11])
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, 1, k)[0]
    qw, codes, s16, z = oracle_packed(w16, bits, g)
    what = oracle.dequantize(codes, s16, z, g)
    check_tol(host(qlin.gemv(qw, dev(x16))), x16, what, str(cfg))
    for kk in (0, 37, k - 64, k - 1):
        e = np.zeros(k, np.float16)
        e[kk] = 1
        ye = host(qlin.gemv(qw, dev(e)))
        assert np.array_equal(ye.astype(np.float64), what[:, kk]), f"{cfg} one-hot k={kk}"


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8, 16])
@pytest.mark.parametrize("group", [64, "K"])
@pytest.mark.parametrize("shape", [(896, 896), (200, 192), (1, 64), (1024, 2048)])
def test_gemv_fused(bits, group, shape):
    if bits == 16 and group == "K":
        pytest.skip("bits=16 has no groups")
    n, k = shape
    g = k if group == "K" else 64
    say(f"gemv fused bits={bits} group={g} shape={shape}")
    rng = np.random.default_rng(3 * n + k + bits)
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, 1, k)[0]
    wd = dev(w16)
    if bits == 16:
        qw = qlin.master_weight(wd, 16, g)
        what = w16.astype(np.float64)
    else:
        s16, z = oracle.rtn_scale_zero(w16, bits, g)
        qw = qlin.master_weight(wd, bits, g, dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
        what = oracle.fused_weights(w16, s16, z, bits, g)
    y = host(qlin.gemv(qw, dev(x16)))
    check_tol(y, x16, what, "fused")
    for kk in sorted({0, k // 3, k - 1}):
        e = np.zeros(k, np.float16)
        e[kk] = 1
        ye = host(qlin.gemv(qw, dev(e)))
        assert np.array_equal(ye.astype(np.float64), what[:, kk]), f"one-hot k={kk}"


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_gemv_fused_edge_groups_exact(bits):
    """Every implicit code of the fused kernel, on groups full of exact ties,
    clamps, constant and one-signed groups: one-hot x over all 256 columns."""
    rng = np.random.default_rng(500 + bits)
    w16 = synth.edge_groups(bits, rng, n_rows=64, k=256)
    say(f"gemv fused edge groups bits={bits}")
    s16, z = oracle.rtn_scale_zero(w16, bits, 64)
    what = oracle.fused_weights(w16, s16, z, bits, 64)
    qw = qlin.master_weight(dev(w16), bits, 64, dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
    eye = torch.eye(256, dtype=torch.float16, device=DEV)
    got = np.stack([host(qlin.gemv(qw, eye[i].contiguous())) for i in range(256)], axis=1)
    assert np.array_equal(got.astype(np.float64), what)


def test_gemv_fused_scale_sweep():
    """The fused kernel's rounding for many (w, s) pairs: every finite fp16 w
    against a spread of fp16 scales, 8-bit with zero 128 (codes -128..127),
    read back through one-hot x.  Compares with the oracle's codes."""
    allw = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allw = allw[np.isfinite(allw)]
    n = ((allw.size + 63) // 64) * 64
    w16 = np.zeros((n, 64), np.float16)
    w16[: allw.size, 0] = allw
    scales = np.array([2.0 ** -14, 2.0 ** -10, 0.00123, 0.0078125, 0.01, 0.0333, 0.125, 0.3,
                       1.0, 1.5, 3.0, 7.0, 100.0, 1000.0], np.float16)
    e = np.zeros(64, np.float16)
    e[0] = 1
    ed = dev(e)
    wd = dev(w16)
    z = np.full((n, 1), 128, np.uint8)
    for s in scales:
        say(f"fused scale sweep s={float(s)}")
        s16 = np.full((n, 1), s, np.float16)
        qw = qlin.master_weight(wd, 8, 64, dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
        got = host(qlin.gemv(qw, ed)).astype(np.float64)
        want = oracle.fused_weights(w16, s16, z, 8, 64)[:, 0]
        assert np.array_equal(got, want), f"s={float(s)}"


# fused launch shapes "waves,splits,rows": whole tiles, 8-row work-groups
FUSED_WIDTHS = ["8,1,64", "4,4,64", "8,1,8", "16,2,8", "4,3,8"]


@pytest.mark.parametrize("bits", [2, 3, 4, 8, 16])
@pytest.mark.parametrize("shape", [(200, 192), (130, 4096), (1, 64)])
@pytest.mark.parametrize("cfg", FUSED_WIDTHS)
def test_gemv_fused_row_widths(bits, shape, cfg, launch_override):
    """The fused kernel at every work-group width and split: within tolerance,
    one-hot x at positions covering every 8-weight slice of the first and last
    block exact."""
    launch_override("gemv", cfg)
    n, k = shape
    say(f"gemv fused cfg={cfg} bits={bits} shape={shape}")
    rng = np.random.default_rng([n, k, bits, 9])
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, 1, k)[0]
    wd = dev(w16)
    if bits == 16:
        qw = qlin.master_weight(wd, 16, 64)
        what = w16.astype(np.float64)
    else:
        s16, z = oracle.rtn_scale_zero(w16, bits, 64)
        qw = qlin.master_weight(wd, bits, 64, dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
        what = oracle.fused_weights(w16, s16, z, bits, 64)
    check_tol(host(qlin.gemv(qw, dev(x16))), x16, what, cfg)
    for kk in sorted(set(range(0, 64, 7)) | set(range(k - 64, k, 9))):
        e = np.zeros(k, np.float16)
        e[kk] = 1
        ye = host(qlin.gemv(qw, dev(e)))
        assert np.array_equal(ye.astype(np.float64), what[:, kk]), f"{cfg} one-hot k={kk}"


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("cfg", ["8,1,64", "8,1,8"])
def test_gemv_fused_edge_groups_widths(bits, cfg, launch_override):
    """Edge-case groups (ties, clamps, constant, one-signed) through both
    fused kernels: one-hot x over all 256 columns, exact."""
    launch_override("gemv", cfg)
    rng = np.random.default_rng(520 + bits)
    w16 = synth.edge_groups(bits, rng, n_rows=64, k=256)
    say(f"gemv fused edge groups cfg={cfg} bits={bits}")
    s16, z = oracle.rtn_scale_zero(w16, bits, 64)
    what = oracle.fused_weights(w16, s16, z, bits, 64)
    qw = qlin.master_weight(dev(w16), bits, 64, dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
    eye = torch.eye(256, dtype=torch.float16, device=DEV)
    got = np.stack([host(qlin.gemv(qw, eye[i].contiguous())) for i in range(256)], axis=1)
    assert np.array_equal(got.astype(np.float64), what)


@pytest.mark.parametrize("cfg", ["8,1,64", "8,1,8"])
def test_gemv_fused_scale_sweep_all_columns(cfg, launch_override):
    """Every finite fp16 weight spread over all 64 columns of a block (so every
    lane slice of the narrow kernel sees them), 8-bit, zero 128, six scales,
    read back column by column through one-hot x."""
    launch_override("gemv", cfg)
    allw = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allw = allw[np.isfinite(allw)]
    n = (allw.size + 63) // 64
    flat = np.zeros(n * 64, np.float16)
    flat[: allw.size] = allw
    w16 = flat.reshape(n, 64)
    wd = dev(w16)
    z = np.full((n, 1), 128, np.uint8)
    eye = torch.eye(64, dtype=torch.float16, device=DEV)
    for s in np.array([2.0 ** -10, 0.00123, 0.125, 1.0, 7.0, 1000.0], np.float16):
        say(f"fused scale sweep cfg={cfg} s={float(s)}")
        s16 = np.full((n, 1), s, np.float16)
        qw = qlin.master_weight(wd, 8, 64, dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
        got = np.stack([host(qlin.gemv(qw, eye[i].contiguous())) for i in range(64)], axis=1)
        want = oracle.fused_weights(w16, s16, z, 8, 64)
        assert np.array_equal(got.astype(np.float64), want), f"s={float(s)}"


# ------------------------------------------------------------------ GEMM --
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("m", [1, 5, 8, 16, 17, 64, 100, 128, 256])
def test_gemm(bits, m):
    n, k = (320, 896) if m != 100 else (200, 192)
    say(f"gemm bits={bits} m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 13 + bits)
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, m, k)
    qw, codes, s16, z = oracle_packed(w16, bits, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    Y = host(qlin.gemm(qw, dev(x16)))
    check_tol(Y, x16, what, f"gemm m={m}")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("m", [1, 5, 16])
def test_gemm_skinny_forced(bits, m, launch_override):
    """The skinny (M <= 16) kernel, forced: within tolerance and one-hot exact."""
    launch_override("gemm", "16,1")
    n, k = 200, 640
    rng = np.random.default_rng([bits, m, 13])
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, m, k)
    qw, codes, s16, z = oracle_packed(w16, bits, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    say(f"gemm skinny forced bits={bits} m={m}")
    check_tol(host(qlin.gemm(qw, dev(x16))), x16, what, f"skinny m={m}")
    cols = (np.arange(m) * 53 + 7) % k
    X = np.zeros((m, k), np.float16)
    X[np.arange(m), cols] = 1
    Y = host(qlin.gemm(qw, dev(X)))
    assert np.array_equal(Y.astype(np.float64), fp16_rne(what[:, cols].T))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("m", [16, 128])
def test_gemm_one_hot_fp16_exact(bits, m):
    """X rows one-hot: Y[i, :] is column k_i of the dequantized weights rounded
    to fp16 (nearest even) -- every decoded weight checked exactly."""
    n, k = 192, 256
    rng = np.random.default_rng(900 + bits + m)
    w16 = synth.edge_groups(bits, rng, n_rows=n, k=k)
    qw, codes, s16, z = oracle_packed(w16, bits, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    say(f"gemm one-hot bits={bits} m={m}")
    for start in range(0, k, m):
        cols = np.arange(start, min(k, start + m))
        X = np.zeros((cols.size, k), np.float16)
        X[np.arange(cols.size), cols] = 1
        Y = host(qlin.gemm(qw, dev(X)))
        assert np.array_equal(Y.astype(np.float64), fp16_rne(what[:, cols].T))


# K-split GEMM launch shapes "0,splits" (32 X rows x one 64-row W tile per
# work-group, its 4 waves splitting K), with and without a K split across
# work-groups
# "mb,splits": K-split with 32 (0) / 64 (1) X rows, over tile pairs of one
# matrix with 64 (2) / 32 (3) X rows (sets run these as 1 / 0), and over half
# tiles with 32 (4) / 64 (5) X rows
KSPLIT = ["0,1", "0,2", "0,5", "1,1", "1,3", "2,1", "2,3", "3,1", "3,2", "4,1", "4,3", "5,1",
          "5,2", "6,1", "6,3", "7,1", "7,2"]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("cfg", KSPLIT)
@pytest.mark.parametrize("m,n,k,group", [(1, 200, 192, 64), (5, 130, 1600, 64), (16, 64, 896, "K"),
                                         (17, 200, 192, 64), (100, 130, 1600, 64),
                                         (100, 130, 2368, 64), (128, 320, 896, "K"),
                                         (256, 64, 4096, 64)])
def test_gemm_ksplit(bits, cfg, m, n, k, group, launch_override):
    """The K-split GEMM within tolerance on ragged M and N, per-group and
    per-channel scales, and one-hot X rows reproduce fp16-rounded dequantized
    columns exactly (every decoded weight of the columns hit).  Grids of at
    most one work-group per CU with long K per wave take the double-buffered
    loop: 37 K-blocks leave the waves 10, 9, 9 and 9 blocks, so the last
    operand set of each wave is partly past the range."""
    launch_override("gemm", cfg)
    g = k if group == "K" else 64
    rng = np.random.default_rng([m, n, k, bits, 11])
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, m, k)
    qw, codes, s16, z = oracle_packed(w16, bits, g)
    what = oracle.dequantize(codes, s16, z, g)
    say(f"gemm ksplit cfg={cfg} bits={bits} m={m} n={n} k={k} group={g}")
    check_tol(host(qlin.gemm(qw, dev(x16))), x16, what, f"ksplit {cfg}")
    cols = (np.arange(m) * 37) % k
    X = np.zeros((m, k), np.float16)
    X[np.arange(m), cols] = 1
    Y = host(qlin.gemm(qw, dev(X)))
    assert np.array_equal(Y.astype(np.float64), fp16_rne(what[:, cols].T))


@pytest.mark.parametrize("bits", [3, 4, 6])
@pytest.mark.parametrize("cfg", KSPLIT)
def test_gemm_ksplit_sets_and_workspace(bits, cfg, launch_override):
    """A ragged set of three matrices in one K-split launch, an explicit
    workspace reused twice (counters re-armed, partial region scratch)."""
    launch_override("gemm", cfg)
    rng = np.random.default_rng([bits, 12])
    k, m = 1024, 72
    mats = []
    for n in (200, 64, 1):
        w16 = synth.master_weights(rng, n, k)
        qw, codes, s16, z = oracle_packed(w16, bits, 64)
        mats.append((qw, oracle.dequantize(codes, s16, z, 64)))
    x16 = synth.activations(rng, m, k)
    need = qlin.library().qlin_gemm_multi_workspace_bytes(
        (qlin.QlinWeightC * 3)(*[q.c_struct() for q, _ in mats]), 3, m)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    say(f"gemm ksplit set cfg={cfg} bits={bits} ws={need}")
    Ys = [host(y) for y in qlin.gemm_multi([q for q, _ in mats], dev(x16), ws=ws)]
    for Y, (_, what) in zip(Ys, mats):
        check_tol(Y, x16, what, f"set {cfg}")
    if need > 65536:
        assert torch.count_nonzero(ws[:65536]).item() == 0
        ws[65536:].fill_(0x5A)
    Ys2 = [host(y) for y in qlin.gemm_multi([q for q, _ in mats], dev(x16), ws=ws)]
    for a, b in zip(Ys, Ys2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("m,n,k", [(2048, 8192, 192), (1100, 12288, 128), (2048, 4096, 256),
                                   (1000, 4160, 320), (300, 256, 960)])
def test_gemm_tile_heights(bits, m, n, k):
    """Large grids select the 128-row X tiles (LDS pipeline, 3 stages), mid
    ones 64 rows (4 stages), small ones 32 rows (register-staged); ragged M and
    N in the last work-groups."""
    say(f"gemm tile heights bits={bits} m={m} n={n} k={k}")
    rng = np.random.default_rng(m + n + k + bits)
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, m, k)
    qw, codes, s16, z = oracle_packed(w16, bits, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    Y = host(qlin.gemm(qw, dev(x16)))
    check_tol(Y, x16, what, f"gemm {m}x{n}x{k}")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("m", [512, 1024])
def test_gemm_lds_one_hot_fp16_exact(bits, m):
    """The 64- and 128-row X tiles (n = 16384 fills the chip): X row i = e_(i mod k)
    gives Y[i, :] = column (i mod k) of the dequantized weights, fp16-rounded."""
    n, k = 16384, 256
    rng = np.random.default_rng(950 + bits + m)
    w16 = synth.edge_groups(bits, rng, n_rows=n, k=k)
    qw, codes, s16, z = oracle_packed(w16, bits, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    say(f"gemm lds one-hot bits={bits} m={m}")
    cols = np.arange(m) % k
    X = np.zeros((m, k), np.float16)
    X[np.arange(m), cols] = 1
    Y = host(qlin.gemm(qw, dev(X)))
    assert np.array_equal(Y.astype(np.float64), fp16_rne(what[:, cols].T))


def test_gemm_group_k_and_strides():
    rng = np.random.default_rng(4)
    n, k, m = 130, 512, 40
    w16 = synth.master_weights(rng, n, k)
    Xfull = synth.activations(rng, m, k + 64)
    qw, codes, s16, z = oracle_packed(w16, 4, k)
    what = oracle.dequantize(codes, s16, z, k)
    Xd = dev(Xfull)[:, :k]
    Yfull = torch.full((m, n + 10), -7.0, device=DEV)
    say("gemm strided, group=k")
    qlin.gemm(qw, Xd, Yfull[:, :n])
    Y = host(Yfull)
    check_tol(Y[:, :n], Xfull[:, :k], what, "strided")
    assert np.all(Y[:, n:] == -7.0)


# ----------------------------------------------------- split-K, determinism
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_split_k_paths(bits):
    n, k = 192, 16384
    rng = np.random.default_rng(60 + bits)
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, 8, k)
    qw, codes, s16, z = oracle_packed(w16, bits, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    need = qlin.library().qlin_gemv_workspace_bytes(qw.c_struct())
    assert need > 0
    say(f"split-K gemv bits={bits}")
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    y_split = host(qlin.gemv(qw, dev(x16[0]), ws=ws))
    y_one = host(qlin.gemv(qw, dev(x16[0]), ws=None))
    check_tol(y_split, x16[0], what, "split")
    check_tol(y_one, x16[0], what, "nosplit")
    counters = ws[:65536]
    assert torch.count_nonzero(counters).item() == 0, "arrival counters must be re-armed to zero"
    ws[65536:].fill_(0x5A)                             # partials are scratch: garbage is fine
    y_again = host(qlin.gemv(qw, dev(x16[0]), ws=ws))
    assert np.array_equal(y_split, y_again)
    say(f"split-K skinny gemm bits={bits}")
    Y = host(qlin.gemm(qw, dev(x16)))
    check_tol(Y, x16, what, "split gemm")
    Y2 = host(qlin.gemm(qw, dev(x16), ws=None))
    check_tol(Y2, x16, what, "nosplit gemm")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("cfg", ["2,1", "2,3", "3,1", "3,2"])
def test_gemm_ksplit_pairable_set(bits, cfg, launch_override):
    """A set whose matrices all have an even tile count (4, 2, 2: the
    Qwen2.5-0.5B q/k/v form) runs over tile pairs: within tolerance, and one-hot
    X rows reproduce every matrix's fp16-rounded columns exactly."""
    launch_override("gemm", cfg)
    rng = np.random.default_rng([bits, 13])
    k, m = 640, 90
    mats = []
    for n in (200, 128, 100):
        w16 = synth.master_weights(rng, n, k)
        qw, codes, s16, z = oracle_packed(w16, bits, 64)
        mats.append((qw, oracle.dequantize(codes, s16, z, 64)))
    x16 = synth.activations(rng, m, k)
    say(f"gemm ksplit pairable set cfg={cfg} bits={bits}")
    Ys = [host(y) for y in qlin.gemm_multi([q for q, _ in mats], dev(x16))]
    for Y, (_, what) in zip(Ys, mats):
        check_tol(Y, x16, what, f"pairable set {cfg}")
    cols = (np.arange(m) * 37) % k
    X = np.zeros((m, k), np.float16)
    X[np.arange(m), cols] = 1
    for Y, (_, what) in zip(qlin.gemm_multi([q for q, _ in mats], dev(X)), mats):
        assert np.array_equal(host(Y).astype(np.float64), fp16_rne(what[:, cols].T))


@pytest.mark.parametrize("bits", [3, 4, 6])
def test_split_k_full_tiles(bits):
    """GEMV with K split across work-groups of whole 64-row tiles (many tiles,
    long K): within tolerance, counters re-armed, partial region scratch."""
    n, k = 2560, 8192
    rng = np.random.default_rng(62 + bits)
    w16 = synth.master_weights(rng, n, k)
    x16 = synth.activations(rng, 1, k)[0]
    qw, codes, s16, z = oracle_packed(w16, bits, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    need = qlin.library().qlin_gemv_workspace_bytes(qw.c_struct())
    assert need > 65536, "this shape is expected to split K"
    say(f"split-K gemv, 64-row tiles, bits={bits}")
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    y = host(qlin.gemv(qw, dev(x16), ws=ws))
    check_tol(y, x16, what, "split")
    assert torch.count_nonzero(ws[:65536]).item() == 0
    ws[65536:].fill_(0x5A)
    assert np.array_equal(y, host(qlin.gemv(qw, dev(x16), ws=ws)))
    check_tol(host(qlin.gemv(qw, dev(x16), ws=None)), x16, what, "nosplit")


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("m,n,k", [(128, 896, 4864), (100, 192, 4096), (256, 1024, 2048),
                                   (40, 300, 1600)])
@pytest.mark.parametrize("cfg", [None, "32,3"])
def test_gemm_tiles_split_k(bits, m, n, k, cfg, launch_override):
    """GEMM with K split across work-groups (uneven last split, tiles past n in
    the last work-group; the default K-split kernel and the 32-row tiled one)
    equals the unsplit launch to tolerance, re-arms its counters, and ignores
    whatever the partial region held before."""
    if cfg is not None:
        launch_override("gemm", cfg)
    rng = np.random.default_rng([61, bits, m, n, k])
    w16 = synth.master_weights(rng, n, k)
    X = synth.activations(rng, m, k)
    qw, codes, s16, z = oracle_packed(w16, bits, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    need = qlin.library().qlin_gemm_workspace_bytes(qw.c_struct(), m)
    assert need > 65536, "this shape is expected to split K"
    say(f"tiled split-K gemm bits={bits} m={m} n={n} k={k} ws={need}")
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    Xd = dev(X)
    Y = host(qlin.gemm(qw, Xd, ws=ws))
    check_tol(Y, X, what, "split")
    assert torch.count_nonzero(ws[:65536]).item() == 0, "arrival counters must be re-armed"
    ws[65536:].fill_(0x5A)
    Y2 = host(qlin.gemm(qw, Xd, ws=ws))
    assert np.array_equal(Y, Y2)
    Y1 = host(qlin.gemm(qw, Xd, ws=None))
    check_tol(Y1, X, what, "nosplit")


def test_shared_workspace_across_shapes():
    """One workspace reused by calls of different shapes and kinds."""
    rng = np.random.default_rng(2)
    cases = [(320, 896, 1), (512, 8192, 1), (128, 4864, 8), (896, 4864, 1), (64, 1024, 16)]
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    say("shared workspace")
    for rep in range(2):
        for (n, k, m) in cases:
            w16 = synth.master_weights(rng, n, k)
            x16 = synth.activations(rng, m, k)
            qw, codes, s16, z = oracle_packed(w16, 4, 64)
            what = oracle.dequantize(codes, s16, z, 64)
            if m == 1:
                y = host(qlin.gemv(qw, dev(x16[0]), ws=ws))
                check_tol(y, x16[0], what, f"shared ws gemv {n}x{k}")
            else:
                Y = host(qlin.gemm(qw, dev(x16), ws=ws))
                check_tol(Y, x16, what, f"shared ws gemm {n}x{k} m={m}")
    assert torch.count_nonzero(ws[:65536]).item() == 0


def test_deterministic():
    rng = np.random.default_rng(1)
    w16 = synth.master_weights(rng, 2048, 4096)
    x16 = synth.activations(rng, 128, 4096)
    qw, _, _, _ = oracle_packed(w16, 4, 64)
    say("determinism")
    xd = dev(x16)
    a = [host(qlin.gemv(qw, xd[0])) for _ in range(3)]
    b = [host(qlin.gemm(qw, xd[:8])) for _ in range(3)]
    c = [host(qlin.gemm(qw, xd)) for _ in range(3)]
    for r in (a, b, c):
        assert all(np.array_equal(r[0], v) for v in r[1:])
