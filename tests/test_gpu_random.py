"""Seeded random cases through every entry point, at the launch shapes the
library picks by default, against the CPU oracle.

Each case draws its own bit width (2..8), grouping (64-code groups or one
group per row), ragged n, k (a multiple of 64 up to 2560), M and, for the
sets, the matrix count and their n.  The fixed tests pin chosen shapes and
every forced kernel form; these reach the policy's choices (narrow or whole
tiles, K split or not, K-split / tiled / LDS GEMM, half tiles, tile pairs)
on shapes nobody picked.  Bars: quantizer codes, scales and zeros bit-exact;
every product within 1e-3 * max_row sum |x w|; SwiGLU outputs within the
bound that tolerance implies (oracle.swiglu_tolerance), plus fp16 rounding
for the fp16 output.
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
KINDS = ("quantize", "gemv", "fused", "gemv_multi", "gemv_swiglu", "gemm", "gemm_multi",
         "gemm_swiglu")
CASES = 320


def say(msg):
    print(msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def packed(w16, bits, g):
    codes, s16, z = oracle.quantize(w16, bits, g)
    n, k = w16.shape
    words = oracle.pack_codes(codes, bits).view(np.int32)
    qw = qlin.QWeight(n, k, bits, g, qlin.FMT_PACKED, dev(words),
                      dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
    return qw, oracle.dequantize(codes, s16, z, g)


def within(y, x16, what, label):
    ref = oracle.matmul_ref(x16, what)
    t = oracle.tolerance_scale(x16, what)
    err = float(np.max(np.abs(y.astype(np.float64) - ref))) if ref.size else 0.0
    assert err <= TOL * t, f"{label}: max err {err:.3e} > {TOL} * {t:.3e}"


def swiglu_within(h16, x16, wg, wu, label):
    ref = oracle.swiglu_ref(x16, wg, wu)
    bound = oracle.swiglu_tolerance(x16, wg, wu) + np.abs(ref) * 2.0 ** -11 + 2.0 ** -25
    err = np.abs(h16.astype(np.float64) - ref)
    assert np.all(err <= bound), f"{label}: max excess {float(np.max(err - bound)):.3e}"


@pytest.mark.parametrize("case", range(CASES))
def test_random_case(case, launch_override):
    launch_override("gemv", None)
    launch_override("gemm", None)
    rng = np.random.default_rng([97, case])
    kind = KINDS[case % len(KINDS)]
    bits = int(rng.integers(2, 9))
    k = 64 * int(rng.integers(1, 41))
    per_row = bool(rng.integers(0, 4) == 0)
    g = k if per_row else 64
    n = int(rng.integers(1, 701))
    m = 1 if kind in ("gemv", "fused", "gemv_multi", "gemv_swiglu") else int(
        rng.choice([int(rng.integers(2, 17)), int(rng.integers(17, 301))]))
    label = f"case {case} {kind} bits={bits} group={g} n={n} k={k} m={m}"
    say(label)
    if kind == "quantize":
        w16 = synth.master_weights(rng, n, k)
        qw = qlin.quantize(dev(w16), bits, g)
        codes, s16, z = oracle.quantize(w16, bits, g)
        assert np.array_equal(host(qw.data).view(np.uint32),
                              oracle.pack_codes(codes, bits).view(np.uint32)), label
        assert np.array_equal(host(qw.scale).view(np.uint16),
                              oracle.tile_meta(s16).view(np.uint16)), label
        assert np.array_equal(host(qw.zero), oracle.tile_meta(z)), label
        return
    x16 = synth.activations(rng, m, k)
    if kind == "fused":
        w16 = synth.master_weights(rng, n, k)
        s16, z = oracle.rtn_scale_zero(w16, bits, g)
        qw = qlin.master_weight(dev(w16), bits, g, dev(oracle.tile_meta(s16)),
                                dev(oracle.tile_meta(z)))
        what = oracle.fused_weights(w16, s16, z, bits, g)
        within(host(qlin.gemv(qw, dev(x16[0]))), x16[0], what, label)
    elif kind in ("gemv", "gemm"):
        qw, what = packed(synth.master_weights(rng, n, k), bits, g)
        if kind == "gemv":
            within(host(qlin.gemv(qw, dev(x16[0]))), x16[0], what, label)
        else:
            within(host(qlin.gemm(qw, dev(x16))), x16, what, label)
    elif kind in ("gemv_multi", "gemm_multi"):
        count = int(rng.integers(2, 5))
        ns = [n] + [int(rng.integers(1, 401)) for _ in range(count - 1)]
        mats = [packed(synth.master_weights(rng, ni, k), bits, g) for ni in ns]
        if kind == "gemv_multi":
            ys = qlin.gemv_multi([q for q, _ in mats], dev(x16[0]))
            for i, (y, (_, what)) in enumerate(zip(ys, mats)):
                within(host(y), x16[0], what, f"{label} matrix {i} n={ns[i]}")
        else:
            Ys = qlin.gemm_multi([q for q, _ in mats], dev(x16))
            for i, (Y, (_, what)) in enumerate(zip(Ys, mats)):
                within(host(Y), x16, what, f"{label} matrix {i} n={ns[i]}")
    else:
        gate, wg = packed(synth.master_weights(rng, n, k), bits, g)
        up, wu = packed(synth.master_weights(rng, n, k), bits, g)
        if kind == "gemv_swiglu":
            _, h16 = qlin.gemv_swiglu(gate, up, dev(x16[0]), want_h=False)
            swiglu_within(host(h16), x16[0], wg, wu, label)
        else:
            _, H16 = qlin.gemm_swiglu(gate, up, dev(x16), want_h=False)
            swiglu_within(host(H16), x16, wg, wu, label)


LARGE_M_CASES = 36


@pytest.mark.parametrize("case", range(LARGE_M_CASES))
def test_random_case_large_m(case, launch_override):
    """Prefill sizes (M = 257 .. 2048), where the policy picks among the
    LDS-pipeline, tiled and K-split GEMMs by grid size."""
    launch_override("gemm", None)
    rng = np.random.default_rng([98, case])
    kind = ("gemm", "gemm_multi", "gemm_swiglu")[case % 3]
    bits = int(rng.integers(2, 9))
    k = 64 * int(rng.integers(1, 17))
    g = k if rng.integers(0, 4) == 0 else 64
    n = int(rng.integers(1, 1601))
    m = int(rng.integers(257, 2049))
    label = f"large-M case {case} {kind} bits={bits} group={g} n={n} k={k} m={m}"
    say(label)
    x16 = synth.activations(rng, m, k)
    if kind == "gemm":
        qw, what = packed(synth.master_weights(rng, n, k), bits, g)
        within(host(qlin.gemm(qw, dev(x16))), x16, what, label)
    elif kind == "gemm_multi":
        ns = [n, int(rng.integers(1, 401))]
        mats = [packed(synth.master_weights(rng, ni, k), bits, g) for ni in ns]
        Ys = qlin.gemm_multi([q for q, _ in mats], dev(x16))
        for i, (Y, (_, what)) in enumerate(zip(Ys, mats)):
            within(host(Y), x16, what, f"{label} matrix {i} n={ns[i]}")
    else:
        gate, wg = packed(synth.master_weights(rng, n, k), bits, g)
        up, wu = packed(synth.master_weights(rng, n, k), bits, g)
        _, H16 = qlin.gemm_swiglu(gate, up, dev(x16), want_h=False)
        swiglu_within(host(H16), x16, wg, wu, label)
