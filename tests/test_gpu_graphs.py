"""The launches the benchmark replays from HIP graphs give, on every replay,
bitwise what the same calls give eagerly: split-K GEMV / GEMM (workspace
counters re-armed in the graph), multi-matrix and SwiGLU GEMV, multi-matrix
GEMM and batched quantization; eager work and synchronizations run between
the replays."""
import numpy as np
import pytest
import torch

import synth
from group_wise_bit_amd import qlin

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_graph_replays_match_eager():
    rng = np.random.default_rng(101)
    k = 8192
    masters = [dev(synth.master_weights(rng, n, k)) for n in (640, 128, 128, 1024, 1024)]
    qs = qlin.quantize_batch(masters, 4, 64)
    x = dev(synth.activations(rng, 1, k)[0])
    X = dev(synth.activations(rng, 8, k))
    X2 = dev(synth.activations(rng, 100, k))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    ys = [torch.empty(w.n, device=DEV) for w in qs[:3]]
    y1 = torch.empty(qs[0].n, device=DEV)
    h = torch.empty(1024, device=DEV)
    h16 = torch.empty(1024, dtype=torch.float16, device=DEV)
    Y8 = [torch.empty(8, w.n, device=DEV) for w in qs[:3]]
    Y100 = torch.empty(100, qs[3].n, device=DEV)
    meta = qlin.quantize_batch(masters, 3, "K", codes=False)

    def calls():
        qlin.gemv(qs[0], x, y1, ws=ws)                       # split K (5 tiles, 128 blocks)
        qlin.gemv_multi(qs[:3], x, ys, ws=ws)
        qlin.gemv_swiglu(qs[3], qs[4], x, h, h16, ws=ws)
        qlin.gemm_multi(qs[:3], X, Y8, ws=ws)                # skinny, split K
        qlin.gemm(qs[3], X2, Y100, ws=ws)                    # tiled, split K
        qlin.quantize_batch(masters, 3, "K", codes=False, outs=meta)

    def outputs():
        torch.cuda.synchronize()
        return [t.clone() for t in [y1, *ys, h, h16, *Y8, Y100] + [m.scale for m in meta] +
                [m.zero for m in meta]]

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        calls()
    s.synchronize()
    eager = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    for rep in range(4):
        for t in [y1, *ys, h, h16, *Y8, Y100]:
            t.fill_(float("nan"))
        for m in meta:
            m.scale.fill_(0)
            m.zero.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        got = outputs()
        for a, b in zip(eager, got):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}"
        # eager work between replays, on the same workspace
        qlin.gemv(qs[0], x, torch.empty_like(y1), ws=ws)
        torch.cuda.synchronize()
    assert torch.count_nonzero(ws[:65536]).item() == 0
