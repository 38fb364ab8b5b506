"""GPU parity at the measured workloads' full sizes, in the launch configuration
bench.py times (the same calls, a 64 MB workspace), checked on sampled whole
64-row tiles that the oracle computes on its own:

* 896x896 int4 g64, seed 0: every output and every code;
* the Qwen2.5-0.5B decode step: all 169 matrices (incl. the 151936x896 LM
  head) quantized on the GPU, codes/scales/zeros of sampled tiles bit-exact,
  GEMV rows of sampled tiles within tolerance;
* prefill GEMMs at M = 128 and 2048 on the layer shapes, and the gate/up
  pair with the SwiGLU epilogue;
* the Qwen3-0.6B fused re-quantization sweep (bits 8/4/3/2, per-group and
  per-channel) on all 196 matrices for two settings and on two layers for all;
* Qwen3-8B layer shapes at int4 and int3 for M = 1, 8, 128, and its gate/up
  pair with the SwiGLU epilogue at M = 8 and 128.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from group_wise_bit_amd import qlin

pytestmark = pytest.mark.gpu
DEV = "cuda"
WS_BYTES = 64 << 20


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def ws():
    return torch.zeros(WS_BYTES, dtype=torch.uint8, device=DEV)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def sample_tiles(n, rng, extra=1):
    t = (n + 63) // 64
    pick = {0, t - 1, t // 2}
    pick |= set(int(v) for v in rng.integers(0, t, size=extra))
    return sorted(pick)


def tile_rows(t, n):
    return np.arange(64 * t, min(64 * t + 64, n))


def check_tol(y, x16, what, label):
    ref = oracle.matmul_ref(x16, what)
    tol = oracle.tolerance_scale(x16, what)
    err = float(np.max(np.abs(y.astype(np.float64) - ref)))
    assert err <= 1e-3 * tol, f"{label}: max err {err:.3e} > 1e-3 * {tol:.3e}"


def check_quantized_tiles(qw, w16, bits, group, tiles):
    """Packed words, scales and zeros of whole tiles equal the oracle's."""
    n, k = w16.shape
    kb = k // 64
    g = 1 if group == k else kb
    wpt = kb * 64 * 2 * bits
    words = qw.data.cpu().numpy().view(np.uint32)
    scale = qw.scale.cpu().numpy().view(np.uint16)
    zero = qw.zero.cpu().numpy()
    for t in tiles:
        rows = tile_rows(t, n)
        codes, s16, z = oracle.quantize(w16[rows], bits, group)
        assert np.array_equal(words[t * wpt:(t + 1) * wpt], oracle.pack_codes(codes, bits)), \
            f"codes of tile {t}"
        ms = oracle.tile_meta(s16).view(np.uint16)
        mz = oracle.tile_meta(z)
        assert np.array_equal(scale[t * g * 64:(t + 1) * g * 64], ms), f"scales of tile {t}"
        assert np.array_equal(zero[t * g * 64:(t + 1) * g * 64], mz), f"zeros of tile {t}"


def test_single_decode_gemv_full(ws):
    w16, x16 = synth.single_gemv_case(0)
    say("896x896 int4 g64 seed 0")
    qw = qlin.quantize(dev(w16), 4, 64)
    codes, s16, z = oracle.quantize(w16, 4, 64)
    assert np.array_equal(qw.data.cpu().numpy().view(np.uint32), oracle.pack_codes(codes, 4))
    y = qlin.gemv(qw, dev(x16), ws=ws).cpu().numpy()
    check_tol(y, x16, oracle.dequantize(codes, s16, z, 64), "896x896")


def test_qwen25_decode_step_full(ws):
    rng = np.random.default_rng(0)
    shapes = synth.qwen25_decode_shapes()
    say(f"Qwen2.5-0.5B decode step: {len(shapes)} matrices")
    for (l, nm, n, k) in shapes:
        w16 = synth.master_weights(synth.layer_rng(1, l, nm), n, k)
        x16 = synth.activations(synth.act_rng(1, l, nm), 1, k)[0]
        qw = qlin.quantize(dev(w16), 4, 64)
        y = qlin.gemv(qw, dev(x16), ws=ws).cpu().numpy()
        tiles = sample_tiles(n, rng, extra=2 if nm == "lm_head" else 0)
        if l in (0, 23) or nm == "lm_head":
            check_quantized_tiles(qw, w16, 4, 64, tiles)
        rows = np.concatenate([tile_rows(t, n) for t in tiles])
        codes, s16, z = oracle.quantize(w16[rows], 4, 64)
        check_tol(y[rows], x16, oracle.dequantize(codes, s16, z, 64), f"layer {l} {nm}")


@pytest.mark.parametrize("m", [128, 2048])
def test_qwen25_prefill_full(ws, m):
    rng = np.random.default_rng(m)
    X = synth.activations(np.random.default_rng([7, m]), m, 4864)
    Xd = dev(X)
    for (l, nm, n, k) in [s for s in synth.qwen25_decode_shapes(False) if s[0] in (0, 11)]:
        say(f"prefill M={m} layer {l} {nm} {n}x{k}")
        w16 = synth.master_weights(synth.layer_rng(1, l, nm), n, k)
        qw = qlin.quantize(dev(w16), 4, 64)
        Y = qlin.gemm(qw, Xd[:, :k], ws=ws).cpu().numpy()
        rows = np.concatenate([tile_rows(t, n) for t in sample_tiles(n, rng)])
        codes, s16, z = oracle.quantize(w16[rows], 4, 64)
        check_tol(Y[:, rows], X[:, :k], oracle.dequantize(codes, s16, z, 64),
                  f"M={m} {nm}")


@pytest.mark.parametrize("m", [128, 2048])
def test_qwen25_prefill_swiglu_full(ws, m):
    """The prefill step's gate/up launch (qlin_gemm_swiglu, fp16 h only, as
    bench.py calls it): sampled tiles of h within the SwiGLU bound."""
    rng = np.random.default_rng([9, m])
    n, k = 4864, 896
    X = synth.activations(np.random.default_rng([7, m]), m, k)
    wg16 = synth.master_weights(synth.layer_rng(1, 0, "gate"), n, k)
    wu16 = synth.master_weights(synth.layer_rng(1, 0, "up"), n, k)
    say(f"prefill gate/up SwiGLU M={m}")
    gate, up = qlin.quantize(dev(wg16), 4, 64), qlin.quantize(dev(wu16), 4, 64)
    _, H16 = qlin.gemm_swiglu(gate, up, dev(X), ws=ws, want_h=False)
    h16 = H16.cpu().numpy()
    rows = np.concatenate([tile_rows(t, n) for t in sample_tiles(n, rng)])
    wg = oracle.dequantize(*oracle.quantize(wg16[rows], 4, 64), 64)
    wu = oracle.dequantize(*oracle.quantize(wu16[rows], 4, 64), 64)
    ref = oracle.swiglu_ref(X, wg, wu)
    bound = oracle.swiglu_tolerance(X, wg, wu) + np.abs(ref) * 2.0 ** -11 + 2.0 ** -25
    err = np.abs(h16[:, rows].astype(np.float64) - ref)
    assert np.all(err <= bound), f"M={m}: max err {err.max():.3e}"


def _fused_case(ws, l, nm, n, k, bits, grp, rng):
    w16 = synth.master_weights(synth.layer_rng(3, l, nm), n, k)
    x16 = synth.activations(synth.act_rng(3, l, nm), 1, k)[0]
    g = 64 if grp == "g64" else k
    wd = dev(w16)
    meta = qlin.quantize(wd, bits, g, codes=False)
    fw = qlin.master_weight(wd, bits, g, meta.scale, meta.zero)
    y = qlin.gemv(fw, dev(x16), ws=ws).cpu().numpy()
    rows = np.concatenate([tile_rows(t, n) for t in sample_tiles(n, rng)])
    s16, z = oracle.rtn_scale_zero(w16[rows], bits, g)
    # the GPU's scale/zero of these rows equal the oracle's
    G = k // g
    sc = meta.scale.cpu().numpy().view(np.uint16)
    idx = np.array([((r // 64) * G + gg) * 64 + r % 64 for r in rows for gg in range(G)])
    assert np.array_equal(sc[idx].reshape(len(rows), G), s16.view(np.uint16)), f"scales {nm}"
    what = oracle.fused_weights(w16[rows], s16, z, bits, g)
    check_tol(y[rows], x16, what, f"fused b={bits} {grp} layer {l} {nm}")


@pytest.mark.parametrize("bits,grp", [(4, "g64"), (2, "row")])
def test_qwen3_06b_fused_all_matrices(ws, bits, grp):
    rng = np.random.default_rng(bits)
    shapes = synth.qwen3_06b_shapes()
    say(f"Qwen3-0.6B fused b={bits} {grp}: {len(shapes)} matrices")
    for (l, nm, n, k) in shapes:
        _fused_case(ws, l, nm, n, k, bits, grp, rng)


@pytest.mark.parametrize("bits", [8, 4, 3, 2])
@pytest.mark.parametrize("grp", ["g64", "row"])
def test_qwen3_06b_fused_sweep_two_layers(ws, bits, grp):
    rng = np.random.default_rng(10 + bits)
    for (l, nm, n, k) in [s for s in synth.qwen3_06b_shapes() if s[0] in (0, 27)]:
        say(f"Qwen3-0.6B fused b={bits} {grp} layer {l} {nm}")
        _fused_case(ws, l, nm, n, k, bits, grp, rng)


@pytest.mark.parametrize("bits", [4, 3])
def test_qwen3_8b_layer_full(ws, bits):
    rng = np.random.default_rng(20 + bits)
    for (l, nm, n, k) in [s for s in synth.qwen3_8b_shapes() if s[0] == 0]:
        say(f"Qwen3-8B b={bits} {nm} {n}x{k}")
        w16 = synth.master_weights(synth.layer_rng(5, l, nm), n, k)
        X = synth.activations(synth.act_rng(5, l, nm), 128, k)
        qw = qlin.quantize(dev(w16), bits, 64)
        tiles = sample_tiles(n, rng)
        check_quantized_tiles(qw, w16, bits, 64, tiles)
        rows = np.concatenate([tile_rows(t, n) for t in tiles])
        codes, s16, z = oracle.quantize(w16[rows], bits, 64)
        what = oracle.dequantize(codes, s16, z, 64)
        Xd = dev(X)
        y = qlin.gemv(qw, Xd[0].contiguous(), ws=ws).cpu().numpy()
        check_tol(y[rows], X[0], what, f"{nm} M=1")
        for m in (8, 128):
            Y = qlin.gemm(qw, Xd[:m], ws=ws).cpu().numpy()
            check_tol(Y[:, rows], X[:m], what, f"{nm} M={m}")


@pytest.mark.parametrize("bits", [4, 3])
def test_qwen3_8b_swiglu_full(ws, bits):
    """The 12288x4096 gate/up pair with the SwiGLU epilogue at M = 8 and 128
    (the grouped M = 8 step's launch): sampled tiles of h within the bound."""
    rng = np.random.default_rng(30 + bits)
    n, k = 12288, 4096
    wg16 = synth.master_weights(synth.layer_rng(5, 0, "gate"), n, k)
    wu16 = synth.master_weights(synth.layer_rng(5, 0, "up"), n, k)
    X = synth.activations(synth.act_rng(5, 0, "gate"), 128, k)
    say(f"Qwen3-8B gate/up SwiGLU b={bits}")
    gate, up = qlin.quantize(dev(wg16), bits, 64), qlin.quantize(dev(wu16), bits, 64)
    rows = np.concatenate([tile_rows(t, n) for t in sample_tiles(n, rng)])
    wg = oracle.dequantize(*oracle.quantize(wg16[rows], bits, 64), 64)
    wu = oracle.dequantize(*oracle.quantize(wu16[rows], bits, 64), 64)
    Xd = dev(X)
    for m in (8, 128):
        _, H16 = qlin.gemm_swiglu(gate, up, Xd[:m], ws=ws, want_h=False)
        ref = oracle.swiglu_ref(X[:m], wg, wu)
        bound = oracle.swiglu_tolerance(X[:m], wg, wu) + np.abs(ref) * 2.0 ** -11 + 2.0 ** -25
        err = np.abs(H16.cpu().numpy()[:, rows].astype(np.float64) - ref)
        assert np.all(err <= bound), f"M={m}: max err {err.max():.3e}"
