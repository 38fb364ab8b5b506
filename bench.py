"""Benchmark of the qlin hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--sections decode,qwen3_8b,qwen3_06b]

One step runs every stage of the path once.  Sections and stages (each
bracketed by HIP events on the stream its kernels run on; medians over the K
timed steps):

decode (the metric's workload) -- the linear layers of a Qwen2.5-0.5B decode
step: 24 layers of q 896->896, k/v 896->128, o 896->896, gate/up 896->4864,
down 4864->896 and the tied 151936x896 LM head, 169 matrices, int4 g64,
fp16 masters ~N(0, 0.02), activations ~N(0, 1):
  decode_step      the step's GEMVs as the per-token dispatch list groups
                   them, 97 launches from one HIP graph: per layer q/k/v in
                   one launch (shared x), o, gate/up with the SwiGLU
                   combination (fp16 h), down reading h; then the LM head.
                   The packed weights rotate over 4 copies (1.08 GB, more
                   than four times the 256 MB Infinity Cache) so they come
                   from HBM
  decode_gemv      the same 169 matrices as 169 separate packed GEMVs
  prefill_step_m128  the 168 layer matrices at M = 128 grouped as the dispatch
                   list groups them: per layer q/k/v in one launch, o, gate/up
                   in one launch with the SwiGLU combination (fp16 h), down
                   reading h (96 launches); fp16 MFMA, fp32 accumulate
  prefill_step_m2048 the same at M = 2048
  prefill_m128     the 168 layer GEMMs as separate launches, M = 128
  prefill_m2048    the same at M = 2048
  gemm_m8          169 GEMMs at M = 8
  fused_gemv       169 fused quantize-dequantize GEMVs from the fp16 masters
  rtn_precompute   scale/zero of all 169 masters (a change of bit width),
                   batched: 64 matrices per launch
  quantize_pack    scale/zero and packed codes of all 169 masters, batched
  lm_head_int8     the tied 151936x896 table at 8 bits, g64: LM-head GEMV
  embed_gather     the same table: one token's embedding row, dequantized to
                   fp16 (a latency figure)
qwen3_8b -- 36 layers of q 4096->4096, k/v 4096->1024, o 4096->4096,
gate/up 4096->12288, down 12288->4096 (252 matrices, 3.8 GB at int4):
  q8_step_int4 / _int3 / _int2     the 252 GEMVs grouped as in decode_step:
                                   144 launches (graph)
  q8_decode_int4 / _int3 / _int2   252 packed GEMVs (graph)
  q8_m8_int4 / _int3               252 GEMMs at M = 8
  q8_m8_step_int4 / _int3          the same grouped as in decode_step: per
                                   layer q/k/v in one launch, o, gate/up with
                                   the SwiGLU epilogue (fp16 h), down reading
                                   h (144 launches)
  q8_m128_int4 / _int3             252 GEMMs at M = 128
qwen3_06b -- the 196 fp16 masters of Qwen3-0.6B (28 layers of q 1024->2048,
k/v 1024->1024, o 2048->1024, gate/up 1024->3072, down 3072->1024):
  q06_fused_b{8..2}_{g64,row}      196 fused GEMVs after a lever move
  q06_lever_b{8..2}_{g64,row}      a lever move: scale/zero of the 196 masters,
                                   64 per launch
  q06_fp16_control                 196 plain fp16 GEMVs (bits = 16)
  q06_packed_b{8..2}               196 packed GEMVs at each width of the lever
                                   (g64, copies rotated past the caches)

`value` is decode_step's weight-stream rate: algorithmic bytes (packed codes,
fp16 scales, uint8 zeros, x, y, h) / decode-step time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
HEADLINE = "q8_step_int4"
FP16_MFMA_PEAK_TFLOPS = 2500.0
ROTATE = 4
C1_CALLS = 64
PEAK_READ_BYTES = 4 << 30
PEAK_MFMA_ITERS = 4096
HERE = os.path.dirname(os.path.abspath(__file__))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--sections", default="decode,qwen3_8b,qwen3_06b,peaks")
    p.add_argument("--phases", default="all",
                   help="comma list of stages to run (default: all of the chosen sections)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a plain device-to-device copy of BYTES bytes five times "
                        "(reference for scaling HBM traffic counters), then exit")
    return p.parse_args()


def copy_calibration(nbytes):
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)


def wbytes(n, k, bits, group):
    """Algorithmic bytes of one packed weight: codes + fp16 scale + uint8 zero."""
    g = k if group == "row" else 64
    return n * k * bits // 8 + n * (k // g) * 3


class Phase:
    def __init__(self, name, run, unit, amount, launches, peak, bound, kernel):
        self.name, self.run, self.unit, self.amount = name, run, unit, amount
        self.launches, self.peak, self.bound, self.kernel = launches, peak, bound, kernel
        self.ms = []


def capture(torch, qlin, call_lists, ws):
    """One HIP graph per list of (weight, x, y) GEMV calls."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for calls in call_lists:
            for w, x, y in calls:
                qlin.gemv(w, x, y, ws=ws)
    stream.synchronize()
    graphs = []
    for calls in call_lists:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for w, x, y in calls:
                qlin.gemv(w, x, y, ws=ws)
        g.keepalive = calls           # the tensors the graph's kernels address
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def capture_calls(torch, call_lists):
    """One HIP graph per list of zero-argument launch functions."""
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for calls in call_lists:
            for f in calls:
                f()
    stream.synchronize()
    graphs = []
    for calls in call_lists:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for f in calls:
                f()
        # The launch functions hold (as default arguments and closures) every
        # tensor the graph's kernels address.  They must outlive the graph:
        # each later capture empties torch's cache, so a tensor freed here
        # would be returned to the driver and a replay would fault.
        g.keepalive = calls
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def grouped_step_calls(qlin, shapes, weights, xs, dev, torch, ws, bits=4):
    """The decode step's linear layers as the per-token dispatch list groups
    them: per layer one launch for q/k/v (shared x), o, one gate/up launch with
    the SwiGLU combination (fp16 h), and down reading that h; then the LM head.
    Returns (launch functions, algorithmic bytes, launches)."""
    idx = {(l, nm): i for i, (l, nm, _, _) in enumerate(shapes)}
    layers = sorted(set(l for (l, nm, _, _) in shapes if nm != "lm_head"))
    calls, nbytes = [], 0
    for l in layers:
        q, k, v, o, g, u, d = (idx[(l, nm)] for nm in ("q", "k", "v", "o", "gate", "up", "down"))
        ys = [torch.empty(shapes[i][2], dtype=torch.float32, device=dev) for i in (q, k, v)]
        yo = torch.empty(shapes[o][2], dtype=torch.float32, device=dev)
        h16 = torch.empty(shapes[g][2], dtype=torch.float16, device=dev)
        yd = torch.empty(shapes[d][2], dtype=torch.float32, device=dev)
        wq, wk, wv, wo, wg, wu, wd = (weights[i] for i in (q, k, v, o, g, u, d))
        calls += [
            lambda wq=wq, wk=wk, wv=wv, x=xs[q], ys=ys: qlin.gemv_multi([wq, wk, wv], x, ys, ws=ws),
            lambda wo=wo, x=xs[o], y=yo: qlin.gemv(wo, x, y, ws=ws),
            lambda wg=wg, wu=wu, x=xs[g], h16=h16: qlin.gemv_swiglu(wg, wu, x, None, h16, ws=ws,
                                                                     want_h=False),
            lambda wd=wd, h16=h16, y=yd: qlin.gemv(wd, h16, y, ws=ws),
        ]
        kk = shapes[q][3]
        nbytes += sum(wbytes(shapes[i][2], shapes[i][3], bits, 64) for i in (q, k, v, o, g, u, d))
        nbytes += 2 * kk + 4 * sum(shapes[i][2] for i in (q, k, v))          # qkv: x, y
        nbytes += 2 * shapes[o][3] + 4 * shapes[o][2]                         # o
        nbytes += 2 * shapes[g][3] + 2 * shapes[g][2]                         # gate/up: x, h16
        nbytes += 2 * shapes[d][3] + 4 * shapes[d][2]                         # down: h16, y
    lm = next((i for i, (_, nm, _, _) in enumerate(shapes) if nm == "lm_head"), None)
    if lm is not None:
        ylm = torch.empty(shapes[lm][2], dtype=torch.float32, device=dev)
        calls.append(lambda w=weights[lm], x=xs[lm], y=ylm: qlin.gemv(w, x, y, ws=ws))
        nbytes += (wbytes(shapes[lm][2], shapes[lm][3], bits, 64) + 2 * shapes[lm][3] +
                   4 * shapes[lm][2])
    return calls, nbytes, len(calls)


def build_decode(torch, qlin, synth, dev, ws, phases, state):
    shapes = synth.qwen25_decode_shapes()              # 169 (layer, name, N, K)
    layer_idx = [i for i, s in enumerate(shapes) if s[1] != "lm_head"]
    t0 = time.time()
    masters = [torch.from_numpy(synth.master_weights(synth.layer_rng(1, l, nm), n, k)).to(dev)
               for (l, nm, n, k) in shapes]
    xs = [torch.from_numpy(synth.activations(synth.act_rng(1, l, nm), 1, k)[0]).to(dev)
          for (l, nm, n, k) in shapes]
    print(f"[bench] decode-step masters generated in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)
    packed = [[qlin.quantize(w, 4, 64) for w in masters] for _ in range(ROTATE)]
    scratch = [qlin.quantize(w, 4, 64) for w in masters]
    meta = [qlin.quantize(w, 4, 64, codes=False) for w in masters]
    fused = [qlin.master_weight(w, 4, 64, m.scale, m.zero) for w, m in zip(masters, meta)]
    ys = [torch.empty(n, dtype=torch.float32, device=dev) for (_, _, n, _) in shapes]
    kmax = max(k for *_, k in shapes)
    nmax = max(n for _, _, n, _ in shapes)
    X = {m: torch.from_numpy(synth.activations(np.random.default_rng([7, m]), m, kmax)).to(dev)
         for m in (8, 128, 2048)}
    Y = {m: torch.empty(m * nmax, dtype=torch.float32, device=dev) for m in (8, 128, 2048)}

    def gemm(w, m):
        # X rows keep their pitch kmax; Y is packed [m, n]
        qlin.gemm(w, X[m][:, : w.k], Y[m][: m * w.n].view(m, w.n), ws=ws)

    lm_idx = next(i for i, (_, nm, _, _) in enumerate(shapes) if nm == "lm_head")
    lm8, ids, y_lm = [], None, None
    if "lm_head_int8" in phases or "embed_gather" in phases:
        # the tied table at 8 bits (NEXT-2 of the path): LM-head GEMV + row gather
        lm8 = [qlin.quantize(masters[lm_idx], 8, 64) for _ in range(ROTATE)]
        ids = torch.tensor([12345], dtype=torch.int32, device=dev)
        y_lm = torch.empty(shapes[lm_idx][2], dtype=torch.float32, device=dev)

    graphs = []
    if "decode_gemv" in phases:
        graphs = capture(torch, qlin, [list(zip(packed[r], xs, ys)) for r in range(ROTATE)], ws)
    grouped, grp_bytes, grp_launches = [], 0, 0
    if "decode_step" in phases:
        lists = []
        for r in range(ROTATE):
            calls, grp_bytes, grp_launches = grouped_step_calls(qlin, shapes, packed[r], xs, dev,
                                                                torch, ws)
            lists.append(calls)
        grouped = capture_calls(torch, lists)

    # Every other stage is one HIP graph per weight rotation as well, so the
    # timed region holds the GPU work only (no per-launch host overhead).
    def per_rotation(make):
        return capture_calls(torch, [make(r) for r in range(ROTATE)])

    staged = {}
    # prefill as the dispatch list groups it: per layer q/k/v (one launch), o,
    # gate/up (one launch), down
    idx = {(l, nm): i for i, (l, nm, _, _) in enumerate(shapes)}
    layers = sorted(set(l for (l, nm, _, _) in shapes if nm != "lm_head"))
    Yg = {}
    for m in (128, 2048):
        if f"prefill_step_m{m}" not in phases:
            continue
        Yg[m] = {nm: torch.empty(m, shapes[idx[(0, nm)]][2], dtype=torch.float32, device=dev)
                 for nm in ("q", "k", "v", "o", "down")}
        Yg[m]["h16"] = torch.empty(m, shapes[idx[(0, "gate")]][2], dtype=torch.float16,
                                   device=dev)

        def step_calls(r, m=m):
            Xm = X[m]
            calls = []
            for l in layers:
                w = {nm: packed[r][idx[(l, nm)]] for nm in ("q", "k", "v", "o", "gate", "up", "down")}
                k1 = w["q"].k
                calls += [
                    lambda w=w, m=m, k1=k1: qlin.gemm_multi(
                        [w["q"], w["k"], w["v"]], Xm[:, :k1],
                        [Yg[m]["q"], Yg[m]["k"], Yg[m]["v"]], ws=ws),
                    lambda w=w, m=m, k1=k1: qlin.gemm(w["o"], Xm[:, :k1], Yg[m]["o"], ws=ws),
                    lambda w=w, m=m, k1=k1: qlin.gemm_swiglu(
                        w["gate"], w["up"], Xm[:, :k1], None, Yg[m]["h16"], ws=ws,
                        want_h=False),
                    lambda w=w, m=m: qlin.gemm(w["down"], Yg[m]["h16"], Yg[m]["down"], ws=ws),
                ]
            return calls
        staged[f"prefill_step_m{m}"] = per_rotation(step_calls)
    for m in (128, 2048):
        if f"prefill_m{m}" in phases:
            staged[f"prefill_m{m}"] = per_rotation(
                lambda r, m=m: [lambda w=packed[r][i], m=m: gemm(w, m) for i in layer_idx])
    if "gemm_m8" in phases:
        staged["gemm_m8"] = per_rotation(lambda r: [lambda w=w: gemm(w, 8) for w in packed[r]])
    if "fused_gemv" in phases:
        staged["fused_gemv"] = capture_calls(torch, [[
            lambda w=w, x=x, y=y: qlin.gemv(w, x, y, ws=ws) for w, x, y in zip(fused, xs, ys)]])
    if "rtn_precompute" in phases:
        staged["rtn_precompute"] = capture_calls(torch, [[
            lambda: qlin.quantize_batch(masters, 4, 64, codes=False, outs=meta)]])
    if "quantize_pack" in phases:
        staged["quantize_pack"] = capture_calls(torch, [[
            lambda: qlin.quantize_batch(masters, 4, 64, outs=scratch)]])
    if "lm_head_int8" in phases:
        staged["lm_head_int8"] = per_rotation(
            lambda r: [lambda w=lm8[r]: qlin.gemv(w, xs[lm_idx], y_lm, ws=ws)])
    if "embed_gather" in phases:
        staged["embed_gather"] = per_rotation(lambda r: [lambda w=lm8[r]: qlin.embed_rows(w, ids)])

    # the single 896x896 int4 g64 GEMV (seed 0): 64 back-to-back calls on the
    # same weight from one graph (the weight stays in L2: a latency figure)
    c1 = None
    if "c1_gemv_latency" in phases:
        w0, x0 = synth.single_gemv_case(0)
        c1w = qlin.quantize(torch.from_numpy(w0).to(dev), 4, 64)
        c1x = torch.from_numpy(x0).to(dev)
        c1y = torch.empty(896, dtype=torch.float32, device=dev)
        c1 = (c1w, c1x, c1y)
        staged["c1_gemv_latency"] = capture_calls(torch, [[
            lambda: qlin.gemv(c1w, c1x, c1y, ws=ws) for _ in range(C1_CALLS)]])

    hold = (masters, xs, ys, packed, scratch, meta, fused, X, Y, Yg, lm8, ids, y_lm, c1)

    def run(name):
        assert hold is not None       # every buffer the graphs address stays alive
        r = state["step"] % ROTATE
        if name == "decode_gemv":
            graphs[r].replay()
        elif name == "decode_step":
            grouped[r].replay()
        else:
            g = staged[name]
            g[r % len(g)].replay()

    dec_bytes = sum(wbytes(n, k, 4, 64) + 2 * k + 4 * n for (_, _, n, k) in shapes)
    master_bytes = sum(2 * n * k for (_, _, n, k) in shapes)
    meta_bytes = sum(n * (k // 64) * 3 for (_, _, n, k) in shapes)
    code_bytes = sum(n * k // 2 for (_, _, n, k) in shapes)
    fl = {m: sum(2 * m * shapes[i][2] * shapes[i][3] for i in layer_idx) for m in (128, 2048)}
    out = [
        Phase("decode_step", run, "GB/s", grp_bytes, grp_launches, HBM_PEAK_GBS, "hbm",
              "k_gemv_narrow<4> (q/k/v set, o, gate/up+SwiGLU, down) + k_gemv_packed<4> (LM head)"),
        Phase("decode_gemv", run, "GB/s", dec_bytes, 169, HBM_PEAK_GBS, "hbm",
              "k_gemv_narrow<4> + k_gemv_packed<4> (LM head)"),
        Phase("prefill_step_m128", run, "TFLOP/s", fl[128], 96, FP16_MFMA_PEAK_TFLOPS, "mfma",
              "k_gemm_ksplit<4> (q/k/v set, o, gate/up+SwiGLU pair, down)"),
        Phase("prefill_step_m2048", run, "TFLOP/s", fl[2048], 96, FP16_MFMA_PEAK_TFLOPS,
              "mfma",
              "k_gemm_lds<4, 128> (gate/up+SwiGLU pair), k_gemm_ksplit<4> (q/k/v set, down), k_gemm_tiles<4, 32> (o)"),
        Phase("prefill_m128", run, "TFLOP/s", fl[128], 168, FP16_MFMA_PEAK_TFLOPS, "mfma",
              "k_gemm_ksplit<4>"),
        Phase("prefill_m2048", run, "TFLOP/s", fl[2048], 168, FP16_MFMA_PEAK_TFLOPS, "mfma",
              "k_gemm_lds<4> / k_gemm_tiles<4> / k_gemm_ksplit<4>"),
        Phase("gemm_m8", run, "GB/s",
              sum(wbytes(n, k, 4, 64) + 16 * k + 32 * n for (_, _, n, k) in shapes), 169,
              HBM_PEAK_GBS, "hbm", "k_gemm_ksplit<4> + k_gemm_skinny<4> (down)"),
        Phase("fused_gemv", run, "GB/s",
              master_bytes + meta_bytes + sum(2 * k + 4 * n for (_, _, n, k) in shapes), 169,
              HBM_PEAK_GBS, "hbm", "k_gemv_fused_narrow<4> + k_gemv_fused<4> (LM head)"),
        Phase("rtn_precompute", run, "GB/s", master_bytes + meta_bytes, 3, HBM_PEAK_GBS,
              "hbm", "k_quantize_g64<4> (no codes; 169 matrices in 3 launches)"),
        Phase("quantize_pack", run, "GB/s", master_bytes + meta_bytes + code_bytes, 3,
              HBM_PEAK_GBS, "hbm", "k_quantize_g64<4> (169 matrices in 3 launches)"),
        Phase("lm_head_int8", run, "GB/s",
              wbytes(shapes[lm_idx][2], shapes[lm_idx][3], 8, 64) + 2 * shapes[lm_idx][3] +
              4 * shapes[lm_idx][2], 1, HBM_PEAK_GBS, "hbm", "k_gemv_packed<8>"),
        Phase("embed_gather", run, "GB/s", 896 + 14 * 3 + 2 * 896 + 4, 1, HBM_PEAK_GBS, "hbm",
              "k_embed_rows<8> (one token; latency)"),
        Phase("c1_gemv_latency", run, "GB/s", C1_CALLS * (wbytes(896, 896, 4, 64) + 2 * 896 +
                                                          4 * 896), C1_CALLS, HBM_PEAK_GBS,
              "latency", "896x896 int4 g64 GEMV, seed 0 (L2-resident; us per call)"),
    ]
    return [p for p in out if p.name in phases], shapes


def build_qwen3_8b(torch, qlin, synth, dev, ws, phases):
    """Weights drawn with the device RNG (seeded) for speed: 6.9 G weights."""
    shapes = synth.qwen3_8b_shapes()
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    t0 = time.time()
    packed = {2: [], 3: [], 4: []}
    xs, ys = [], []
    for (l, nm, n, k) in shapes:
        w16 = (torch.randn(n, k, generator=g, device=dev) * 0.02).half()
        for b in packed:
            packed[b].append(qlin.quantize(w16, b, 64))
        xs.append(torch.randn(k, generator=g, device=dev).half())
        ys.append(torch.empty(n, dtype=torch.float32, device=dev))
        del w16
    kmax = max(k for *_, k in shapes)
    nmax = max(n for _, _, n, _ in shapes)
    X = {m: torch.randn(m, kmax, generator=g, device=dev).half() for m in (8, 128)}
    Y = {m: torch.empty(m * nmax, dtype=torch.float32, device=dev) for m in (8, 128)}
    torch.cuda.synchronize()
    print(f"[bench] Qwen3-8B shapes quantized in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    graphs, steps, step_bytes = {}, {}, {}
    for b in (4, 3, 2):
        if f"q8_decode_int{b}" in phases:
            graphs[b] = capture(torch, qlin, [list(zip(packed[b], xs, ys))], ws)[0]
        if f"q8_step_int{b}" in phases:
            calls, step_bytes[b], _ = grouped_step_calls(qlin, shapes, packed[b], xs, dev, torch,
                                                         ws, bits=b)
            steps[b] = capture_calls(torch, [calls])[0]

    gemms = {}
    for b in (4, 3):
        for m in (8, 128):
            if f"q8_m{m}_int{b}" in phases:
                gemms[(b, m)] = capture_calls(torch, [[
                    lambda w=w, m=m: qlin.gemm(w, X[m][:, : w.k], Y[m][: m * w.n].view(m, w.n),
                                               ws=ws) for w in packed[b]]])[0]

    # M = 8 grouped like the decode step; h of the gate/up pair feeds down
    idx = {(l, nm): i for i, (l, nm, _, _) in enumerate(shapes)}
    layers = sorted(set(l for (l, *_) in shapes))
    n_of = {nm: shapes[idx[(0, nm)]][2] for nm in ("q", "k", "v", "o", "gate", "down")}
    Y8 = {nm: torch.empty(8, n_of[nm], dtype=torch.float32, device=dev)
          for nm in ("q", "k", "v", "o", "down")}
    H8 = torch.empty(8, n_of["gate"], dtype=torch.float16, device=dev)
    m8_steps, m8_bytes = {}, {}
    for b in (4, 3):
        if f"q8_m8_step_int{b}" not in phases:
            continue
        calls, nbytes = [], 0
        for l in layers:
            w = {nm: packed[b][idx[(l, nm)]] for nm in ("q", "k", "v", "o", "gate", "up", "down")}
            k1 = w["q"].k
            calls += [
                lambda w=w, k1=k1: qlin.gemm_multi([w["q"], w["k"], w["v"]], X[8][:, :k1],
                                                   [Y8["q"], Y8["k"], Y8["v"]], ws=ws),
                lambda w=w, k1=k1: qlin.gemm(w["o"], X[8][:, :k1], Y8["o"], ws=ws),
                lambda w=w, k1=k1: qlin.gemm_swiglu(w["gate"], w["up"], X[8][:, :k1], None, H8,
                                                    ws=ws, want_h=False),
                lambda w=w: qlin.gemm(w["down"], H8, Y8["down"], ws=ws),
            ]
            # weights + X read once per launch + outputs (fp32 Y, fp16 h)
            nbytes += sum(wbytes(x.n, x.k, b, 64) for x in w.values())
            nbytes += 4 * 16 * k1 + 16 * w["down"].k
            nbytes += 32 * (w["q"].n + w["k"].n + w["v"].n + w["o"].n + w["down"].n)
            nbytes += 16 * w["gate"].n
        m8_steps[b] = capture_calls(torch, [calls])[0]
        m8_bytes[b] = nbytes

    # the step's gate/up SwiGLU launches alone (the dominant kernel of the
    # decode step: 52 % of its bytes), timed on their own for the roofline
    pair_graphs, pair_bytes = {}, {}
    Hp = torch.empty(n_of["gate"], dtype=torch.float16, device=dev)
    for b in (4, 3, 2):
        if f"q8_pair_int{b}" not in phases:
            continue
        calls, nbytes = [], 0
        for l in layers:
            wg, wu = packed[b][idx[(l, "gate")]], packed[b][idx[(l, "up")]]
            x = xs[idx[(l, "gate")]]
            calls.append(lambda wg=wg, wu=wu, x=x: qlin.gemv_swiglu(wg, wu, x, None, Hp, ws=ws,
                                                                    want_h=False))
            nbytes += 2 * wbytes(wg.n, wg.k, b, 64) + 2 * wg.k + 2 * wg.n
        pair_graphs[b] = capture_calls(torch, [calls])[0]
        pair_bytes[b] = nbytes

    # prefill at M = 128 grouped like the decode step: per layer q/k/v (one
    # launch), o, gate/up with the SwiGLU epilogue (fp16 H), down reading H
    Y128 = {nm: torch.empty(128, n_of[nm], dtype=torch.float32, device=dev)
            for nm in ("q", "k", "v", "o", "down")}
    H128 = torch.empty(128, n_of["gate"], dtype=torch.float16, device=dev)
    p128_steps = {}
    for b in (4, 3):
        if f"q8_prefill_step_m128_int{b}" not in phases:
            continue
        calls = []
        for l in layers:
            w = {nm: packed[b][idx[(l, nm)]] for nm in ("q", "k", "v", "o", "gate", "up", "down")}
            k1 = w["q"].k
            calls += [
                lambda w=w, k1=k1: qlin.gemm_multi([w["q"], w["k"], w["v"]], X[128][:, :k1],
                                                   [Y128["q"], Y128["k"], Y128["v"]], ws=ws),
                lambda w=w, k1=k1: qlin.gemm(w["o"], X[128][:, :k1], Y128["o"], ws=ws),
                lambda w=w, k1=k1: qlin.gemm_swiglu(w["gate"], w["up"], X[128][:, :k1], None,
                                                    H128, ws=ws, want_h=False),
                lambda w=w: qlin.gemm(w["down"], H128, Y128["down"], ws=ws),
            ]
        p128_steps[b] = capture_calls(torch, [calls])[0]

    hold = (packed, xs, ys, X, Y, Y8, H8, Hp, Y128, H128)

    def run(name):
        assert hold is not None       # every buffer the graphs address stays alive
        b = int(name[-1])
        if "prefill_step" in name:
            p128_steps[b].replay()
        elif "pair" in name:
            pair_graphs[b].replay()
        elif "m8_step" in name:
            m8_steps[b].replay()
        elif "step" in name:
            steps[b].replay()
        elif "decode" in name:
            graphs[b].replay()
        else:
            gemms[(b, 8 if "_m8_" in name else 128)].replay()

    out = []
    for b in (4, 3, 2):
        out.append(Phase(f"q8_step_int{b}", run, "GB/s", step_bytes.get(b, 0), 144, HBM_PEAK_GBS,
                         "hbm", f"k_gemv_packed<{b}> (q/k/v set, gate/up+SwiGLU, down), k_gemv_narrow<{b}> (o)"))
        out.append(Phase(f"q8_decode_int{b}", run, "GB/s",
                         sum(wbytes(n, k, b, 64) + 2 * k + 4 * n for (_, _, n, k) in shapes),
                         252, HBM_PEAK_GBS, "hbm", f"k_gemv_packed<{b}> + k_gemv_narrow<{b}>"))
        out.append(Phase(f"q8_pair_int{b}", run, "GB/s", pair_bytes.get(b, 0), 36, HBM_PEAK_GBS,
                         "hbm", f"gate/up SwiGLU pair GEMV, 12288x4096 x 2, int{b} (36 launches)"))
    for b in (4, 3):
        out.append(Phase(f"q8_prefill_step_m128_int{b}", run, "TFLOP/s",
                         sum(2 * 128 * n * k for (_, _, n, k) in shapes), 144,
                         FP16_MFMA_PEAK_TFLOPS, "mfma",
                         f"q/k/v set, o, gate/up+SwiGLU pair, down at M = 128, int{b}"))
        out.append(Phase(f"q8_m8_int{b}", run, "GB/s",
                         sum(wbytes(n, k, b, 64) + 16 * k + 32 * n for (_, _, n, k) in shapes),
                         252, HBM_PEAK_GBS, "hbm", f"k_gemm_ksplit<{b}>"))
        out.append(Phase(f"q8_m8_step_int{b}", run, "GB/s", m8_bytes.get(b, 0), 144,
                         HBM_PEAK_GBS, "hbm",
                         f"k_gemm_ksplit<{b}> (q/k/v set, o, gate/up+SwiGLU pair, down)"))
        out.append(Phase(f"q8_m128_int{b}", run, "TFLOP/s",
                         sum(2 * 128 * n * k for (_, _, n, k) in shapes), 252,
                         FP16_MFMA_PEAK_TFLOPS, "mfma", f"k_gemm_ksplit<{b}>"))
    return [p for p in out if p.name in phases]


def build_qwen3_06b(torch, qlin, synth, dev, ws, phases):
    shapes = synth.qwen3_06b_shapes()
    g = torch.Generator(device=dev)
    g.manual_seed(6)
    masters = [(torch.randn(n, k, generator=g, device=dev) * 0.02).half() for (_, _, n, k) in shapes]
    xs = [torch.randn(k, generator=g, device=dev).half() for (_, _, n, k) in shapes]
    ys = [torch.empty(n, dtype=torch.float32, device=dev) for (_, _, n, k) in shapes]
    combos = [(b, gr) for b in (8, 7, 6, 5, 4, 3, 2) for gr in ("g64", "row")]
    meta = {c: [qlin.quantize(w, c[0], 64 if c[1] == "g64" else "K", codes=False) for w in masters]
            for c in combos}
    fused = {c: [qlin.master_weight(w, c[0], 64 if c[1] == "g64" else "K", m.scale, m.zero)
                 for w, m in zip(masters, meta[c])] for c in combos}
    control = [qlin.master_weight(w, 16, 64) for w in masters]
    torch.cuda.synchronize()

    def gemvs(ws_list):
        return [lambda w=w, x=x, y=y: qlin.gemv(w, x, y, ws=ws) for w, x, y in zip(ws_list, xs, ys)]

    staged = {}
    if "q06_fp16_control" in phases:
        staged["q06_fp16_control"] = capture_calls(torch, [gemvs(control)])[0]
    for c in combos:
        tag = f"b{c[0]}_{c[1]}"
        if f"q06_fused_{tag}" in phases:
            staged[f"q06_fused_{tag}"] = capture_calls(torch, [gemvs(fused[c])])[0]
        if f"q06_lever_{tag}" in phases:
            # a lever move: all 196 masters re-quantized, 64 per launch
            staged[f"q06_lever_{tag}"] = capture_calls(torch, [[
                lambda c=c: qlin.quantize_batch(masters, c[0], 64 if c[1] == "g64" else "K",
                                                codes=False, outs=meta[c])]])[0]

    # the packed lever: codes at every width, copies rotated so that one pass
    # set exceeds the 256 MB Infinity Cache several times over
    packed = {}
    for b in (8, 7, 6, 5, 4, 3, 2):
        if f"q06_packed_b{b}" not in phases:
            continue
        per_copy = sum(wbytes(n, k, b, 64) for (_, _, n, k) in shapes)
        copies = max(2, -(-1_100_000_000 // per_copy))
        packed[b] = [qlin.quantize_batch(masters, b, 64) for _ in range(copies)]
        staged[f"q06_packed_b{b}"] = capture_calls(torch, [gemvs(cp) for cp in packed[b]])
    torch.cuda.synchronize()
    turn = {"n": 0}

    hold = (masters, xs, ys, meta, fused, control, packed)

    def run(name):
        assert hold is not None       # every buffer the graphs address stays alive
        g = staged[name]
        if isinstance(g, list):
            turn["n"] += 1
            g[turn["n"] % len(g)].replay()
        else:
            g.replay()

    master_bytes = sum(2 * n * k for (_, _, n, k) in shapes)
    act = sum(2 * k + 4 * n for (_, _, n, k) in shapes)
    out = []
    for (b, gr) in combos:
        mb = sum(n * (k // (64 if gr == "g64" else k)) * 3 for (_, _, n, k) in shapes)
        out.append(Phase(f"q06_fused_b{b}_{gr}", run, "GB/s", master_bytes + mb + act, 196,
                         HBM_PEAK_GBS, "hbm", f"k_gemv_fused_narrow<{b}>"))
        out.append(Phase(f"q06_lever_b{b}_{gr}", run, "GB/s", master_bytes + mb, 4,
                         HBM_PEAK_GBS, "hbm",
                         f"k_quantize_{'g64' if gr == 'g64' else 'row'}<{b}> (no codes)"))
    out.append(Phase("q06_fp16_control", run, "GB/s", master_bytes + act, 196, HBM_PEAK_GBS,
                     "hbm", "k_gemv_fused_narrow<16>"))
    for b in (8, 7, 6, 5, 4, 3, 2):
        out.append(Phase(f"q06_packed_b{b}", run, "GB/s",
                         sum(wbytes(n, k, b, 64) for (_, _, n, k) in shapes) + act, 196,
                         HBM_PEAK_GBS, "hbm", f"k_gemv_narrow<{b}> + k_gemv_packed<{b}>"))
    return [p for p in out if p.name in phases]


def build_peaks(torch, dev, phases):
    """The achieved peaks: a streaming read of 4 GiB (HBM) and a matrix-core
    loop with no memory traffic (fp16 MFMA), from libqlin_peaks.so."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(HERE, "group_wise_bit_amd", "libqlin_peaks.so"))
    lib.qlin_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.qlin_peak_mfma.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.qlin_peak_mfma_waves.restype = ctypes.c_int64
    lib.qlin_peak_read_groups.restype = ctypes.c_int64
    src = torch.ones(PEAK_READ_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(int(lib.qlin_peak_read_groups()), dtype=torch.int32, device=dev)
    waves = int(lib.qlin_peak_mfma_waves())
    fsink = torch.zeros(waves, dtype=torch.float32, device=dev)

    def read():
        st = lib.qlin_peak_stream_read(src.data_ptr(), PEAK_READ_BYTES, sink.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
        assert st == 0, st

    def mfma():
        st = lib.qlin_peak_mfma(PEAK_MFMA_ITERS, fsink.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
        assert st == 0, st
    graphs = {}
    if "peak_stream_read" in phases:
        graphs["peak_stream_read"] = capture_calls(torch, [[read]])[0]
    if "peak_mfma" in phases:
        graphs["peak_mfma"] = capture_calls(torch, [[mfma]])[0]
    hold = (src, sink, fsink, lib)

    def run(name):
        assert hold is not None
        graphs[name].replay()
    out = [Phase("peak_stream_read", run, "GB/s", PEAK_READ_BYTES, 1, HBM_PEAK_GBS, "hbm",
                 "streaming read of 4 GiB, one contiguous chunk per work-group, 16-byte loads (libqlin_peaks)"),
           Phase("peak_mfma", run, "TFLOP/s", waves * PEAK_MFMA_ITERS * 8 * 32768, 1,
                 FP16_MFMA_PEAK_TFLOPS, "mfma",
                 "v_mfma_f32_32x32x16_f16 loop, 8 independent accumulators per wave")]
    return [p for p in out if p.name in phases]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard output rows across GPUs; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    import synth
    from group_wise_bit_amd import qlin

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sections = [s for s in args.sections.split(",") if s]
    want = None if args.phases == "all" else set(p for p in args.phases.split(",") if p)

    def chosen(names):
        return set(names) if want is None else set(names) & want

    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    state = {"step": 0}
    phases, decode_shapes = [], None
    if "decode" in sections:
        names = ["decode_step", "decode_gemv", "prefill_step_m128", "prefill_step_m2048",
                 "prefill_m128", "prefill_m2048", "gemm_m8", "fused_gemv",
                 "rtn_precompute", "quantize_pack", "lm_head_int8", "embed_gather",
                 "c1_gemv_latency"]
        ps, decode_shapes = build_decode(torch, qlin, synth, dev, ws, chosen(names), state)
        phases += ps
    if "qwen3_8b" in sections:
        names = [f"q8_{s}_int{b}" for b in (4, 3, 2) for s in ("step", "decode", "pair")] + [
            f"q8_m{m}_int{b}" for b in (4, 3) for m in (8, 128)] + [
            f"q8_m8_step_int{b}" for b in (4, 3)] + [
            f"q8_prefill_step_m128_int{b}" for b in (4, 3)]
        phases += build_qwen3_8b(torch, qlin, synth, dev, ws, chosen(names))
    if "qwen3_06b" in sections:
        names = ([f"q06_{k}_b{b}_{g}" for k in ("fused", "lever") for b in (8, 7, 6, 5, 4, 3, 2)
                  for g in ("g64", "row")] + ["q06_fp16_control"] +
                 [f"q06_packed_b{b}" for b in (8, 7, 6, 5, 4, 3, 2)])
        phases += build_qwen3_06b(torch, qlin, synth, dev, ws, chosen(names))
    if "peaks" in sections:
        phases += build_peaks(torch, dev, chosen(["peak_stream_read", "peak_mfma"]))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(record):
        for p in phases:
            if record:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
            p.run(p.name)
            if record:
                b.record(stream)
                p.ms.append((a, b))
        state["step"] += 1

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    print(f"[bench] {args.steps} timed steps in {wall:.2f}s", file=sys.stderr, flush=True)

    res, rooflines = {}, {}
    for p in phases:
        ms = np.array([a.elapsed_time(b) for a, b in p.ms])
        med = float(np.median(ms))
        scale = 1e9 if p.unit == "GB/s" else 1e12
        rate = p.amount / (med * 1e-3) / scale
        res[p.name] = {"ms_median": round(med, 4), "ms_p10": round(float(np.percentile(ms, 10)), 4),
                       "ms_p90": round(float(np.percentile(ms, 90)), 4), p.unit: round(rate, 2),
                       "launches": p.launches}
        rooflines[p.name] = {"bound": p.bound, "kernel": p.kernel, "achieved": round(rate, 2),
                             "peak": p.peak, "unit": p.unit, "frac": round(rate / p.peak, 4)}

    head = HEADLINE if HEADLINE in res else None
    out = {
        "metric": "GEMV weight GB/s (% HBM peak) + prefill GEMM TFLOP/s, int4 g64",
        "value": res[head]["GB/s"] if head else None, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": res[head]["ms_median"] if head else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,0.02) fp16 masters, N(0,1) fp16 activations)",
        "config": {"workload": "Qwen3-8B-shaped decode step: 36 layers x {q 4096->4096, k/v "
                               "4096->1024 (q/k/v one launch), o 4096->4096, gate/up "
                               "4096->12288 (one launch, SwiGLU epilogue, fp16 h), down "
                               "12288->4096}, 252 matrices, int4 g64, M=1, 144 launches "
                               "from one HIP graph",
                   "global_batch": 1, "seq_len": 1, "parallelism": "single GPU",
                   "weight_bytes_per_step": [p for p in phases if p.name == head][0].amount
                   if head else None,
                   "sections": sections},
        "loop_ms_per_step": round(wall * 1e3 / args.steps, 4),
    }
    if not args.no_cpu_baseline and "qwen3_8b" in sections:
        out["cpu_baseline"] = cpu_baseline_c5()
    if head is not None:
        out["pct_hbm_peak"] = round(100 * res[head]["GB/s"] / HBM_PEAK_GBS, 2)
    pair = "q8_pair_int4"
    if pair in res:
        ph = [p for p in phases if p.name == pair][0]
        per_launch_us = res[pair]["ms_median"] * 1e3 / ph.launches
        bpl = ph.amount / ph.launches
        achieved = bpl / (per_launch_us * 1e-6) / 1e9
        traffic = measured_traffic()
        out["roofline"] = {
            "bound": "hbm", "kernel": "gate/up SwiGLU pair GEMV of the decode step "
                                      "(2 x 12288x4096 int4 g64 + x + fp16 h; 36 launches)",
            "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": int(bpl), "avg_launch_us": round(per_launch_us, 3),
        }
    tf = {}
    for key, label in (("prefill_step_m2048", "qwen25_M2048_step"),
                       ("prefill_step_m128", "qwen25_M128_step"),
                       ("q8_prefill_step_m128_int4", "qwen3_8b_M128_step"),
                       ("q8_m128_int4", "qwen3_8b_M128_separate")):
        if key in res:
            tf[label] = res[key]["TFLOP/s"]
    if tf:
        out["prefill_gemm_tflops"] = tf
        out["prefill_pct_fp16_mfma_peak"] = {k: round(100 * v / FP16_MFMA_PEAK_TFLOPS, 2)
                                             for k, v in tf.items()}
    peaks = {}
    if "peak_stream_read" in res:
        peaks["stream_read_GBs"] = res["peak_stream_read"]["GB/s"]
    if "peak_mfma" in res:
        peaks["mfma_f16_TFLOPs"] = res["peak_mfma"]["TFLOP/s"]
    if peaks:
        if head is not None and "stream_read_GBs" in peaks:
            peaks["value_pct_of_read"] = round(100 * res[head]["GB/s"] / peaks["stream_read_GBs"], 2)
        if "mfma_f16_TFLOPs" in peaks and tf:
            peaks["prefill_pct_of_mfma_loop"] = {
                k: round(100 * v / peaks["mfma_f16_TFLOPs"], 2) for k, v in tf.items()}
        out["achieved_peaks"] = peaks
    if "c1_gemv_latency" in res:
        out["c1_us_per_call"] = round(res["c1_gemv_latency"]["ms_median"] * 1e3 / C1_CALLS, 3)
    # the per-stage detail last, after every summary key
    out["phases"] = res
    out["rooflines"] = rooflines
    print(json.dumps(out), flush=True)


TRAFFIC_SUMMARY = os.path.join(HERE, "profiles",
                               "gemv_int4_qwen3_8b_gate_up_pair_hbm_traffic.txt")


def kernel_source_hash():
    import glob
    import hashlib
    csrc = os.path.join(HERE, "group_wise_bit_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(csrc, "*.h")) + glob.glob(os.path.join(csrc, "*.hip"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per gate/up pair launch from the committed rocprofv3 counter
    summary, or None when the kernel sources changed after the counters were
    taken."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    vals = dict(line.split(": ", 1) for line in text.splitlines()
                if line.startswith(("kernel source sha256", "traffic_bytes_per_launch")))
    key = [k for k in vals if k.startswith("kernel source sha256")]
    if not key or vals[key[0]].strip() != kernel_source_hash():
        return None
    return float(vals["traffic_bytes_per_launch"])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_c5():
    """The oracle (plain NumPy) on a bounded sample of the headline workload:
    the seven matrices of one Qwen3-8B layer (q, k, v, o, gate, up, down;
    193 M weights) at int4 g64, M = 1.  Three phases timed apart with
    time.perf_counter: quantize (binary32 RTN), dequantize (binary64), matmul
    (binary64 BLAS).  `value` is the oracle's GEMV weight-stream rate in the
    metric's unit: algorithmic weight bytes / (dequantize + matmul) time, on
    all host cores; the same with one BLAS thread is reported beside it.
    (NumPy's elementwise phases run on one thread either way.)"""
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    layer = [(0, nm, n, k) for (l, nm, n, k) in synth.qwen3_8b_shapes() if l == 0]
    mats = []
    for (l, nm, n, k) in layer:
        w16 = synth.master_weights(synth.layer_rng(5, l, nm), n, k)
        x = synth.activations(synth.act_rng(5, l, nm), 1, k)[0]
        mats.append((w16, x, n * k // 2 + n * (k // 64) * 3 + 2 * k + 4 * n))

    def one_pass():
        tq = td = tm = 0.0
        for w16, x, _ in mats:
            t0 = time.perf_counter()
            codes, s16, z = oracle.quantize(w16, 4, 64)
            t1 = time.perf_counter()
            what = oracle.dequantize(codes, s16, z, 64)
            t2 = time.perf_counter()
            oracle.matmul_ref(x, what)
            t3 = time.perf_counter()
            tq, td, tm = tq + t1 - t0, td + t2 - t1, tm + t3 - t2
            del codes, what
        return tq, td, tm
    nbytes = sum(b for *_, b in mats)
    runs = {}
    for label, threads in (("all_cores", cores), ("one_thread", 1)):
        with threadpool_limits(limits=threads):
            tq, td, tm = one_pass()
        runs[label] = {"threads": threads, "quantize_s": round(tq, 3),
                       "dequantize_s": round(td, 3), "matmul_s": round(tm, 3),
                       "GBs": round(nbytes / (td + tm) / 1e9, 4)}
    return {"value": runs["all_cores"]["GBs"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "one Qwen3-8B layer (q, k, v, o, gate, up, down: 193 M weights), int4 "
                      "g64, M = 1; GB/s = weight bytes / (dequantize + matmul); quantize "
                      "timed apart",
            "cpu_model": cpu_model(), "phases": runs}


if __name__ == "__main__":
    main()
