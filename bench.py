"""Benchmark of the qlin hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: the linear layers of a Qwen2.5-0.5B decode step -- 24 layers of
q 896->896, k/v 896->128, o 896->896, gate/up 896->4864, down 4864->896, plus
the tied 151936x896 LM head (169 matrices) -- synthetic fp16 masters
~N(0, 0.02), fp16 activations ~N(0, 1), int4 with groups of 64 along K.

One step runs every stage of the path once over those shapes, each stage
bracketed by HIP events on the stream its kernels run on:
  decode_gemv      169 packed int4 GEMVs (M = 1), replayed from one HIP graph
  prefill_m128     168 GEMMs at M = 128 (layers only; fp16 MFMA, fp32 acc)
  prefill_m2048    168 GEMMs at M = 2048
  gemm_m8          169 GEMMs at M = 8
  fused_gemv       169 fused quantize-dequantize GEMVs from the fp16 masters
  rtn_precompute   scale/zero precompute of all 169 masters (no codes)
  quantize_pack    scale/zero + codes of all 169 masters
The packed weights rotate over 4 copies (>1 GB, four times the 256 MB
Infinity Cache) so the decode stage reads them from HBM, not from cache.

`value` is the decode stage's weight-stream rate: algorithmic bytes (packed
codes + fp16 scales + uint8 zeros + x + y) / decode-stage time.  The prefill
GEMM rate is reported beside it, as the metric asks.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
ROTATE = 4


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--phases", default="all",
                   help="comma list of stages to run (default: all)")
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
    all_phases = ["decode_gemv", "prefill_m128", "prefill_m2048", "gemm_m8", "fused_gemv",
                  "rtn_precompute", "quantize_pack"]
    phases = all_phases if args.phases == "all" else [p for p in args.phases.split(",") if p]

    shapes = synth.qwen25_decode_shapes()              # 169 (layer, name, N, K)
    layer_idx = [i for i, s in enumerate(shapes) if s[1] != "lm_head"]
    t0 = time.time()
    masters = []
    for (l, nm, n, k) in shapes:
        w = synth.master_weights(synth.layer_rng(1, l, nm), n, k)
        masters.append(torch.from_numpy(w).to(dev))
    xs = []
    for (l, nm, n, k) in shapes:
        x = synth.activations(synth.act_rng(1, l, nm), 1, k)[0]
        xs.append(torch.from_numpy(x).to(dev))
    print(f"[bench] masters generated and uploaded in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)

    # packed copies for the decode stage (rotated for a cold Infinity Cache)
    packed = [[qlin.quantize(w, 4, 64) for w in masters] for _ in range(ROTATE)]
    scratch = [qlin.quantize(w, 4, 64) for w in masters]        # target of quantize_pack
    meta = [qlin.quantize(w, 4, 64, codes=False) for w in masters]
    fused = [qlin.master_weight(w, 4, 64, m.scale, m.zero) for w, m in zip(masters, meta)]
    ys = [torch.empty(n, dtype=torch.float32, device=dev) for (_, _, n, _) in shapes]
    kmax = max(k for *_, k in shapes)
    nmax = max(n for _, _, n, _ in shapes)
    X = {m: torch.from_numpy(synth.activations(np.random.default_rng([7, m]), m, kmax)).to(dev)
         for m in (8, 128, 2048)}
    Y = {m: torch.empty(m * nmax, dtype=torch.float32, device=dev) for m in (8, 128, 2048)}
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def gemm(w, m):
        # X rows keep their pitch kmax; Y is packed [m, n]
        qlin.gemm(w, X[m][:, : w.k], Y[m][: m * w.n].view(m, w.n), ws=ws)

    # one HIP graph per packed copy for the decode stage (169 launches each)
    graphs = []
    if "decode_gemv" in phases:
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for r in range(ROTATE):                       # warm the library's device check
                for w, x, y in zip(packed[r], xs, ys):
                    qlin.gemv(w, x, y, ws=ws)
        stream.synchronize()
        for r in range(ROTATE):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for w, x, y in zip(packed[r], xs, ys):
                    qlin.gemv(w, x, y, ws=ws)
            graphs.append(g)
        torch.cuda.synchronize()

    def run_phase(name, step):
        if name == "decode_gemv":
            graphs[step % ROTATE].replay()
        elif name == "prefill_m128":
            for i in layer_idx:
                gemm(packed[step % ROTATE][i], 128)
        elif name == "prefill_m2048":
            for i in layer_idx:
                gemm(packed[step % ROTATE][i], 2048)
        elif name == "gemm_m8":
            for w in packed[step % ROTATE]:
                gemm(w, 8)
        elif name == "fused_gemv":
            for w, x, y in zip(fused, xs, ys):
                qlin.gemv(w, x, y, ws=ws)
        elif name == "rtn_precompute":
            for w, m in zip(masters, meta):
                qlin.quantize(w, 4, 64, codes=False, out=m)
        elif name == "quantize_pack":
            for w, s in zip(masters, scratch):
                qlin.quantize(w, 4, 64, out=s)

    # algorithmic work per stage
    def wbytes(n, k, bits=4, g=64):
        return n * k * bits // 8 + n * (k // g) * 3
    dec_bytes = sum(wbytes(n, k) + 2 * k + 4 * n for (_, _, n, k) in shapes)
    master_bytes = sum(2 * n * k for (_, _, n, k) in shapes)
    meta_bytes = sum(n * (k // 64) * 3 for (_, _, n, k) in shapes)
    code_bytes = sum(n * k // 2 for (_, _, n, k) in shapes)
    fl = {m: sum(2 * m * shapes[i][2] * shapes[i][3] for i in layer_idx) for m in (128, 2048)}
    fl8 = sum(2 * 8 * n * k for (_, _, n, k) in shapes)
    work = {
        "decode_gemv": ("GB/s", dec_bytes),
        "prefill_m128": ("TFLOP/s", fl[128]),
        "prefill_m2048": ("TFLOP/s", fl[2048]),
        "gemm_m8": ("GB/s", sum(wbytes(n, k) + 16 * k + 32 * n for (_, _, n, k) in shapes)),
        "fused_gemv": ("GB/s", master_bytes + meta_bytes + sum(2 * k + 4 * n for (_, _, n, k) in shapes)),
        "rtn_precompute": ("GB/s", master_bytes + meta_bytes),
        "quantize_pack": ("GB/s", master_bytes + meta_bytes + code_bytes),
    }

    stream = torch.cuda.current_stream()
    ev = {p: [] for p in phases}

    def step(i, record):
        for p in phases:
            if record:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
            run_phase(p, i)
            if record:
                b.record(stream)
                ev[p].append((a, b))

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    res = {}
    for p in phases:
        ms = np.array([a.elapsed_time(b) for a, b in ev[p]])
        unit, amount = work[p]
        med = float(np.median(ms))
        rate = amount / (med * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
        res[p] = {"ms_median": round(med, 4), "ms_p10": round(float(np.percentile(ms, 10)), 4),
                  "ms_p90": round(float(np.percentile(ms, 90)), 4), unit: round(rate, 2),
                  "launches": 169 if p in ("decode_gemv", "gemm_m8", "fused_gemv",
                                            "rtn_precompute", "quantize_pack") else 168}

    out = {
        "metric": "GEMV weight GB/s (% HBM peak) + prefill GEMM TFLOP/s, int4 g64",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,0.02) fp16 masters, N(0,1) fp16 activations)",
        "config": {"workload": "Qwen2.5-0.5B decode step linear layers, 169 GEMVs incl. "
                               "151936x896 LM head, int4 g64, M=1",
                   "global_batch": 1, "seq_len": 1, "parallelism": "single GPU",
                   "hip_graph": True, "weight_copies_rotated": ROTATE},
        "phases": res,
    }
    if "decode_gemv" in res:
        gbs = res["decode_gemv"]["GB/s"]
        out["value"] = gbs
        out["pct_hbm_peak"] = round(100 * gbs / HBM_PEAK_GBS, 2)
        per_launch_us = res["decode_gemv"]["ms_median"] * 1e3 / 169
        out["roofline"] = {
            "bound": "hbm", "kernel": "k_gemv_packed<4> (169 launches per step)",
            "achieved": round(dec_bytes / 169 / (per_launch_us * 1e-6) / 1e9, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dec_bytes / 169 / (per_launch_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "algorithmic_bytes_per_launch": dec_bytes / 169,
            "avg_launch_us": round(per_launch_us, 3),
        }
    if "prefill_m2048" in res:
        out["prefill_gemm_tflops"] = {"M=2048": res["prefill_m2048"]["TFLOP/s"]}
        if "prefill_m128" in res:
            out["prefill_gemm_tflops"]["M=128"] = res["prefill_m128"]["TFLOP/s"]
        out["prefill_pct_fp16_mfma_peak"] = round(
            100 * res["prefill_m2048"]["TFLOP/s"] / FP16_MFMA_PEAK_TFLOPS, 2)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shapes)
    print(json.dumps(out), flush=True)


TRAFFIC_SUMMARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "gemv_packed_int4_qwen25_decode_hbm_traffic.txt")


def kernel_source_hash():
    import glob
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "group_wise_bit_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(csrc, "*.h")) + glob.glob(os.path.join(csrc, "*.hip"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    or None when the kernel sources changed after the counters were taken."""
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


def cpu_baseline(shapes, min_seconds=10.0):
    """The oracle (plain NumPy) on the same decode step, in the same unit.

    The oracle's GEMV is dequantize (binary64) + binary64 matmul from the
    codes/scales/zeros its own quantizer produced (quantization not timed).
    It runs over the 169 matrices in order, repeating the step until at least
    `min_seconds` of timed CPU work have accumulated."""
    import oracle
    import synth
    cores = os.cpu_count() or 1
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    prepared = []
    for (l, nm, n, k) in shapes:
        w16 = synth.master_weights(synth.layer_rng(1, l, nm), n, k)
        x = synth.activations(synth.act_rng(1, l, nm), 1, k)[0]
        codes, s16, z = oracle.quantize(w16, 4, 64)
        prepared.append((x, codes, s16, z, n * k // 2 + n * (k // 64) * 3 + 2 * k + 4 * n))
        del w16
    t_total, nbytes, passes = 0.0, 0, 0
    while t_total < min_seconds:
        for (x, codes, s16, z, b) in prepared:
            t = time.perf_counter()
            what = oracle.dequantize(codes, s16, z, 64)
            oracle.matmul_ref(x, what)
            t_total += time.perf_counter() - t
            nbytes += b
        passes += 1
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"the whole 169-matrix decode step, {passes} pass(es), "
                      f"{t_total:.1f} s timed; dequantize + fp64 matmul per matrix, "
                      "codes from the oracle's own quantizer (not timed)"}


if __name__ == "__main__":
    main()
