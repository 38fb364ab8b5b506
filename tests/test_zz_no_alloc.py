"""qlin_gemv_noalloc (the GEMV for callers that cannot allocate): through the
C ABI, its output equals qlin_gemv's with a workspace of the size the library
asks for, bit for bit (the same kernels at the same launch shape), on two
calls in a row, the second with a smaller input; and it refuses a weight
whose split-K workspace would not fit its static scratch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from group_wise_bit_amd import qlin

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def packed(w16, bits, group=64):
    codes, s16, z = oracle.quantize(w16, bits, group)
    n, k = w16.shape
    words = oracle.pack_codes(codes, bits).view(np.int32)
    qw = qlin.QWeight(n, k, bits, group, qlin.FMT_PACKED, dev(words),
                      dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
    return qw, oracle.dequantize(codes, s16, z, group)


def run_pair(qw, x16, what, label):
    print(f"noalloc {label}", flush=True)
    ws = qlin.workspace(int(qlin.library().qlin_gemv_workspace_bytes(ctypes.byref(qw.c_struct()))),
                        torch.device(DEV))
    ref = host(qlin.gemv(qw, dev(x16), ws=ws))
    got = host(qlin.gemv_noalloc(qw, dev(x16)))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), label
    t = oracle.tolerance_scale(x16, what)
    assert np.max(np.abs(got.astype(np.float64) - oracle.matmul_ref(x16, what))) <= 1e-3 * t


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_noalloc_matches_gemv_two_calls(bits):
    rng = np.random.default_rng(100 + bits)
    # first call: a long-K launch that splits K (uses the scratch), then a
    # smaller one
    for n, k in ((4096, 12288), (640, 4864), (200, 192)):
        w16 = synth.master_weights(rng, n, k)
        x16 = synth.activations(rng, 1, k)[0]
        qw, what = packed(w16, bits)
        run_pair(qw, x16, what, f"bits={bits} {n}x{k}")


def test_noalloc_fused_master():
    rng = np.random.default_rng(7)
    w16 = synth.master_weights(rng, 512, 8192)
    x16 = synth.activations(rng, 1, 8192)[0]
    s16, z = oracle.rtn_scale_zero(w16, 4, 64)
    qw = qlin.master_weight(dev(w16), 4, 64, dev(oracle.tile_meta(s16)), dev(oracle.tile_meta(z)))
    run_pair(qw, x16, oracle.fused_weights(w16, s16, z, 4, 64), "fused 512x8192")


def test_noalloc_refuses_oversized_workspace():
    """A launch whose split-K workspace exceeds the 1 MiB scratch is refused
    on the host (sizes only: fake, never dereferenced device addresses)."""
    lib = qlin.library()
    fake = 0x7F0000000000
    # fp16 masters, 256 tiles, K = 65536: 16-way split of 16384 rows
    w = qlin.QlinWeightC(16384, 65536, 4, 64, qlin.FMT_FP16_MASTER, 0, fake, 65536,
                         fake + (1 << 40), fake + (2 << 40))
    assert lib.qlin_gemv_workspace_bytes(ctypes.byref(w)) > (1 << 20)
    assert lib.qlin_gemv_noalloc(ctypes.byref(w), fake + (3 << 40), fake + (4 << 40), None) == 8
