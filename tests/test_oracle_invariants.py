"""Invariants, statistics and byte-accounting pins of the oracle.

* codes stay in [0, 2^bits - 1];
* an unclamped code is within half a scale of its weight (exactly);
* a clamped code is within s/2 + qmax*|s32 - s16| (the fp16 scale may round
  below the binary32 one, Examples F and G in tests/golden);
* quantization noise is uniform: MSE ~= mean(s^2)/12 for 3 bits and up;
* one scale per 64-weight group beats one scale per output channel at the
  same bit width (Bitcrush README, "The machine", NAIVE/SMART row);
* the model byte totals printed on the pages are reproduced from the shape
  tables the bench uses (Bitcrush README, "The machine", BRAIN SIZE row;
  Enargeia, "Run it" and "Measured, not asserted").
"""
import numpy as np
import pytest

import oracle
import synth


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
def test_round_trip_bounds(bits, group):
    rng = np.random.default_rng(bits * 10 + (1 if group == "K" else 0))
    w16 = np.concatenate([synth.master_weights(rng, 96, 512),
                          synth.edge_groups(bits, rng, n_rows=32, k=512)])
    g = 512 if group == "K" else 64
    codes, s16, z = oracle.quantize(w16, bits, g)
    qmax = (1 << bits) - 1
    assert codes.min() >= 0 and codes.max() <= qmax
    what = oracle.dequantize(codes, s16, z, g)
    w = w16.astype(np.float64)
    err = np.abs(w - what)                                   # exact in binary64
    s = np.repeat(s16.astype(np.float64), g, axis=1)
    zz = np.repeat(z.astype(np.int64), g, axis=1)
    # the unrounded code position before clamping (exact rational ties are
    # not an issue here: only the clamped/unclamped split is needed)
    ratio = np.where(s > 0, w / np.where(s > 0, s, 1), 0)
    unclamped = (s > 0) & (ratio + zz >= -0.5) & (ratio + zz <= qmax + 0.5)
    assert np.all(err[unclamped] <= s[unclamped] / 2)
    # clamped: the extreme can sit beyond the grid by qmax*(s32 - s16)
    mn = w.reshape(w.shape[0], -1, g).min(axis=2)
    mx = w.reshape(w.shape[0], -1, g).max(axis=2)
    s32 = ((mx - mn).astype(np.float32) / np.float32(qmax)).astype(np.float64)
    slack = np.repeat(np.abs(s32 - s16.astype(np.float64)) * qmax, g, axis=1)
    normal = (s > 0) & ~unclamped
    # one-signed groups are excluded: their zero point clamps by design
    zeroinside = np.repeat((mn <= 0) & (mx >= 0), g, axis=1)
    sel = normal & zeroinside
    assert np.all(err[sel] <= s[sel] / 2 + slack[sel] + s[sel] * 1e-4)
    # constant groups: everything 0
    assert np.all(what[s == 0] == 0)


@pytest.mark.parametrize("bits", [3, 4, 5, 6, 7, 8])
def test_mse_is_uniform_noise(bits):
    rng = np.random.default_rng(42)
    w16 = synth.master_weights(rng, 512, 1024)
    codes, s16, z = oracle.quantize(w16, bits, 64)
    what = oracle.dequantize(codes, s16, z, 64)
    mse = np.mean((w16.astype(np.float64) - what) ** 2)
    expect = np.mean(s16.astype(np.float64) ** 2) / 12
    assert 0.97 < mse / expect < 1.03


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_per_group_beats_per_channel(bits):
    rng = np.random.default_rng(3)
    w16 = synth.master_weights(rng, 256, 1024)
    errs = {}
    for g in (64, 1024):
        codes, s16, z = oracle.quantize(w16, bits, g)
        errs[g] = np.mean((w16.astype(np.float64) - oracle.dequantize(codes, s16, z, g)) ** 2)
    assert errs[64] < 0.8 * errs[1024]


def test_brain_size_bytes_qwen3_06b():
    linears = sum(n * k for _, _, n, k in synth.qwen3_06b_shapes())
    assert len(synth.qwen3_06b_shapes()) == 196
    rest = synth.QWEN3_06B_EMBED[0] * synth.QWEN3_06B_EMBED[1] + synth.QWEN3_06B_NORM_PARAMS
    assert linears + rest == 596_049_920                    # "596-million-parameter"
    assert 2 * (linears + rest) == 1_192_099_840             # 1,192 MB at fp16
    assert linears * 2 // 8 + 2 * rest == 421_396_480       # 421 MB at 2-bit, no metadata


def test_enargeia_parameter_count():
    linears = sum(n * k for _, _, n, k in synth.qwen25_decode_shapes(include_lm_head=False))
    vocab, hidden = synth.QWEN25_05B_LM_HEAD[1:]
    total = linears + vocab * hidden + synth.QWEN25_05B_EXTRA_PARAMS
    assert total == 494_032_768                            # "494.0M parameters"
    assert round(4 * total / 2 ** 20, 1) == 1884.6          # fp32 MiB
    assert len(synth.qwen25_decode_shapes()) == 169


def test_kv_cache_bytes():
    # 24 layers x (K and V) x 2048 positions x (2 kv heads x 64) x fp16
    assert 24 * 2 * 2048 * 128 * 2 / 2 ** 20 == 24.0
