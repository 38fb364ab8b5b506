"""GPU parity of qlin_embed_rows (the tied embedding table's row gather)
against the oracle's dequantized weights: fp32 rows exactly s*(q - z), fp16
rows exactly those values rounded to nearest even; ids out of range give
zero rows; the int8 g64 table of the Qwen2.5-0.5B shape (151936 x 896)."""
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


def packed(w16, bits, group):
    codes, s16, z = oracle.quantize(w16, bits, group)
    n, k = w16.shape
    words = oracle.pack_codes(codes, bits).view(np.int32)
    qw = qlin.QWeight(n, k, bits, group, qlin.FMT_PACKED, dev(words),
                      dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
    return qw, codes, s16, z


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
def test_embed_rows_exact(bits, group):
    n, k = 1000, 896
    g = k if group == "K" else group
    rng = np.random.default_rng([81, bits, g])
    w16 = synth.edge_groups(bits, rng, n_rows=n, k=k) if bits != 8 else \
        synth.master_weights(rng, n, k)
    qw, codes, s16, z = packed(w16, bits, g)
    ids = np.array([0, n - 1, 5, 5, 63, 64, 999, 500, 17, 0] + list(rng.integers(0, n, 20)),
                   dtype=np.int32)
    say(f"embed rows bits={bits} group={g} count={ids.size}")
    o16, o32 = qlin.embed_rows(qw, dev(ids), want16=True, want32=True)
    torch.cuda.synchronize()
    ref = oracle.dequantize(codes, s16, z, g)[ids]
    assert np.array_equal(o32.cpu().numpy().astype(np.float64), ref)
    ref16 = ref.astype(np.float32).astype(np.float16)      # exact in fp32, then nearest even
    assert np.array_equal(o16.cpu().numpy().view(np.uint16), ref16.view(np.uint16))


def test_embed_rows_out_of_range_and_empty():
    rng = np.random.default_rng(82)
    qw, *_ = packed(synth.master_weights(rng, 130, 192), 4, 64)
    ids = np.array([-1, 130, 2 ** 31 - 1, 3], dtype=np.int32)
    say("embed rows out of range")
    o16, o32 = qlin.embed_rows(qw, dev(ids), want32=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o32[:3]).item() == 0 and torch.count_nonzero(o16[:3]).item() == 0
    assert torch.count_nonzero(o32[3]).item() > 0
    e16, e32 = qlin.embed_rows(qw, dev(np.zeros(0, np.int32)), want32=True)
    assert e16.shape == (0, 192) and e32.shape == (0, 192)


def test_embed_rows_qwen25_int8_table():
    """The tied 151936 x 896 embedding at 8 bits, g64: sampled rows exact, and
    the same packed table serves the LM-head GEMV."""
    n, k = 151936, 896
    w16 = synth.master_weights(synth.layer_rng(1, 24, "lm_head"), n, k)
    say("qwen2.5 int8 tied table")
    qw = qlin.quantize(dev(w16), 8, 64)
    rng = np.random.default_rng(83)
    ids = np.concatenate([[0, n - 1], rng.integers(0, n, 62)]).astype(np.int32)
    o16, o32 = qlin.embed_rows(qw, dev(ids), want32=True)
    torch.cuda.synchronize()
    codes, s16, z = oracle.quantize(w16[ids], 8, 64)
    ref = oracle.dequantize(codes, s16, z, 64)
    assert np.array_equal(o32.cpu().numpy().astype(np.float64), ref)
    assert np.array_equal(o16.cpu().numpy().view(np.uint16),
                          ref.astype(np.float32).astype(np.float16).view(np.uint16))
    # LM head: logits of the gathered x through the same table, sampled rows
    x16 = o16[5].contiguous()
    y = qlin.gemv(qw, x16).cpu().numpy()
    rows = np.sort(rng.integers(0, n, 256))
    c2, s2, z2 = oracle.quantize(w16[rows], 8, 64)
    what = oracle.dequantize(c2, s2, z2, 64)
    xr = x16.cpu().numpy()
    err = np.max(np.abs(y[rows] - oracle.matmul_ref(xr, what)))
    assert err <= 1e-3 * oracle.tolerance_scale(xr, what)
