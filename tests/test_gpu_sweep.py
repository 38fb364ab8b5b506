"""The exhaustive (w, s) sweep, on the GPU, against the oracle.

The rounding of a master to its code -- rint(w / s) + z, clamped -- runs
inside two kernels: the fused re-rounding GEMV (Bitcrush README, "Under the
hood": the codes are computed inline from the fp16 masters with the
precomputed scale and zero) and the quantizer.  Both are checked here for
every finite fp16 weight against every positive fp16 scale:

* Fused GEMV, 8 bits, zero 128: every finite fp16 w (63,488) against every
  positive finite fp16 s (31,743), 2.0e9 pairs, in both fused kernel forms
  (whole 64-row tiles and 8-row work-groups).  A row holds 64 weights and one
  scale; one-hot x reads column c of every row, so y = s * (q - 128), which
  fp32 holds exactly, compared bit for bit with the oracle.
* Quantizer: every reachable positive stored scale (all up to 43680 at
  2 bits, up to 514 at 8 bits; tests/sweep_groups.py realizes each with a
  pair of extremes) with every fp16 value between its extremes, 2.0e9
  masters.  Scales and zero points compared bit for bit; the codes through
  one-hot x as s * (q - z) (exact in fp32; s > 0 fixes q).

Scales go in chunks, in order; the oracle's side of each chunk is computed
ahead in worker threads, and the first mismatch stops the sweep with the
scale and the weight that differ.
"""
import collections
import concurrent.futures as cf
import itertools

import numpy as np
import pytest
import torch

import oracle
import sweep_groups as sg
from group_wise_bit_amd import qlin

pytestmark = pytest.mark.gpu
DEV = "cuda"
WORKERS = 8
FUSED_CHUNK = 512          # scales per chunk: 507,904 rows, 32.5 M pairs
QUANT_CHUNK = 16 << 20     # masters per chunk


def say(msg):
    print(msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def ahead(fn, items, depth=WORKERS + 2):
    """(item, fn(item)) in order, with up to `depth` items computed ahead in
    worker threads (NumPy releases the GIL in its array loops)."""
    with cf.ThreadPoolExecutor(WORKERS) as pool:
        it = iter(items)
        futs = collections.deque((x, pool.submit(fn, x)) for x in itertools.islice(it, depth))
        while futs:
            x, f = futs.popleft()
            res = f.result()
            nxt = next(it, None)
            if nxt is not None:
                futs.append((nxt, pool.submit(fn, nxt)))
            yield x, res


def one_hot_columns(qw, n, eye, Yt):
    """Yt[c, :n] = W_hat[:, c] through 64 one-hot GEMVs; returns [n, 64] on the host."""
    for c in range(64):
        qlin.gemv(qw, eye[c], y=Yt[c, :n])
    torch.cuda.synchronize()
    return Yt[:, :n].cpu().numpy().T


def first_mismatch(got, want):
    bad = np.flatnonzero(got.astype(np.float64).ravel() != want.ravel())
    if bad.size == 0:
        return None
    return np.unravel_index(int(bad[0]), want.shape), int(bad.size)


def test_fused_every_weight_every_scale(launch_override):
    allw = sg.every_finite_fp16().reshape(-1, 64)          # 992 rows of 64
    rps = allw.shape[0]
    scales = sg.every_positive_fp16()
    bounds = [(a, min(a + FUSED_CHUNK, scales.size)) for a in range(0, scales.size, FUSED_CHUNK)]
    W = np.tile(allw, (FUSED_CHUNK, 1))
    wd = dev(W)
    eye = torch.eye(64, dtype=torch.float16, device=DEV)
    Yt = torch.empty((64, W.shape[0]), dtype=torch.float32, device=DEV)

    def expected(ab):
        sc = scales[ab[0]:ab[1]]
        n = sc.size * rps
        s16 = np.repeat(sc, rps)[:, None]
        z = np.full((n, 1), 128, np.uint8)
        return oracle.fused_weights(W[:n], s16, z, 8, 64), s16, z

    pairs = 0
    for (a, b), (want, s16, z) in ahead(expected, bounds):
        n = s16.shape[0]
        sd, zd = dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z))
        for cfg in ("8,1,64", "8,1,8"):
            launch_override("gemv", cfg)
            qw = qlin.master_weight(wd[:n], 8, 64, sd, zd)
            got = one_hot_columns(qw, n, eye, Yt)
            bad = first_mismatch(got, want)
            if bad is not None:
                (r, c), count = bad
                pytest.fail(f"fused {cfg}: {count} mismatches in scales [{a}, {b}); first "
                            f"s={float(s16[r, 0])!r} w={float(W[r, c])!r} "
                            f"got {float(got[r, c])!r} want {float(want[r, c])!r}")
        pairs += want.size
        if a % (8 * FUSED_CHUNK) == 0:
            say(f"fused sweep: scales [{a}, {b}) of {scales.size} ok ({pairs} pairs)")
    assert pairs == scales.size * 63488
    say(f"fused sweep: {pairs} (w, s) pairs, both kernel forms, bit-exact")


@pytest.mark.parametrize("bits", [2, 8])
def test_quantizer_every_reachable_scale(bits, launch_override):
    launch_override("gemv", None)
    scales = sg.every_positive_fp16()
    found, mn, mx = sg.realize_scales(scales, bits)
    idx = np.flatnonzero(found)
    counts = sg.values_between(mn[idx], mx[idx])
    bounds = sg.chunks_by_count(counts, QUANT_CHUNK)
    eye = torch.eye(64, dtype=torch.float16, device=DEV)
    Yt = torch.empty((64, 0), dtype=torch.float32, device=DEV)

    def expected(ab):
        sel = idx[ab[0]:ab[1]]
        W, sidx = sg.quantizer_groups(mn[sel], mx[sel])
        codes, s16, z = oracle.quantize(W, bits, 64)
        assert np.array_equal(s16[:, 0].view(np.uint16), scales[sel][sidx].view(np.uint16))
        return W, sel[sidx], s16, z, oracle.dequantize(codes, s16, z, 64)

    masters = 0
    for i, (_, (W, row_scale, s16, z, want)) in enumerate(ahead(expected, bounds)):
        n = W.shape[0]
        if Yt.shape[1] < n:
            # rows 16-byte aligned: a pitch of whole 64-float lines
            Yt = torch.empty((64, (n + 8192 + 63) // 64 * 64), dtype=torch.float32, device=DEV)
        q = qlin.quantize(dev(W), bits, 64)
        torch.cuda.synchronize()
        gs = q.scale.cpu().numpy().view(np.uint16)[:n]
        gz = q.zero.cpu().numpy()[:n]
        if not np.array_equal(gs, s16[:, 0].view(np.uint16)):
            r = int(np.flatnonzero(gs != s16[:, 0].view(np.uint16))[0])
            pytest.fail(f"{bits}-bit scale of row {r} (target s={float(scales[row_scale[r]])!r}): "
                        f"got {gs[r]:#06x} want {s16[r, 0].view(np.uint16):#06x}")
        if not np.array_equal(gz, z[:, 0]):
            r = int(np.flatnonzero(gz != z[:, 0])[0])
            pytest.fail(f"{bits}-bit zero of row {r} (s={float(s16[r, 0])!r}): "
                        f"got {gz[r]} want {z[r, 0]}")
        got = one_hot_columns(q, n, eye, Yt)
        bad = first_mismatch(got, want)
        if bad is not None:
            (r, c), count = bad
            pytest.fail(f"{bits}-bit codes: {count} mismatches; first s={float(s16[r, 0])!r} "
                        f"z={z[r, 0]} w={float(W[r, c])!r} got {float(got[r, c])!r} "
                        f"want {float(want[r, c])!r}")
        masters += W.size
        if i % 16 == 0:
            say(f"quantizer sweep {bits}-bit: chunk {i + 1} of {len(bounds)} ok "
                f"({masters} masters)")
    assert masters >= int(counts.sum())
    say(f"quantizer sweep {bits}-bit: {idx.size} scales, {masters} masters, bit-exact")
