"""Run one GEMM launch shape a few times, for profiling its kernel alone.

    python -m group_wise_bit_amd.probe WORKLOAD CASE FORM [BITS]

WORKLOAD: q8m128 / q8m8 / q8m2048 (Qwen3-8B layer shapes at M = 128 / 8 /
2048) or q25m2048 (Qwen2.5-0.5B at M = 2048).  CASE: qkv (the q/k/v set),
o, pair (gate/up with the SwiGLU epilogue, fp16 h), down.  FORM: "default"
(the library's launch policy) or "form,splits" for the GEMM launch-shape
override (include/qlin_tune.h).  BITS: 4 by default.

Eight calls over four rotating copies of the weights (int4 g64, N(0, 0.02)
fp16 masters quantized on the device, X ~ N(0, 1)), then one
synchronization; under `rocprofv3 --kernel-trace` or `--pmc` every call is
one dispatch of the chosen kernel.
"""
import sys

import torch

from group_wise_bit_amd import qlin

QWEN3_8B = {'q': (4096, 4096), 'k': (1024, 4096), 'v': (1024, 4096), 'o': (4096, 4096),
            'gate': (12288, 4096), 'up': (12288, 4096), 'down': (4096, 12288)}
QWEN25_05B = {'q': (896, 896), 'k': (128, 896), 'v': (128, 896), 'o': (896, 896),
              'gate': (4864, 896), 'up': (4864, 896), 'down': (896, 4864)}
WORKLOADS = {'q8m128': (QWEN3_8B, 128), 'q8m8': (QWEN3_8B, 8), 'q8m2048': (QWEN3_8B, 2048),
             'q25m2048': (QWEN25_05B, 2048)}
CASES = {'qkv': ['q', 'k', 'v'], 'o': ['o'], 'pair': ['gate', 'up'], 'down': ['down']}


def main(argv):
    if len(argv) < 3 or argv[0] not in WORKLOADS or argv[1] not in CASES:
        print(__doc__)
        return 2
    shapes, m = WORKLOADS[argv[0]]
    case, form = argv[1], argv[2]
    bits = int(argv[3]) if len(argv) > 3 else 4
    mats = CASES[case]
    dev = torch.device('cuda:0')
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    ws = torch.zeros(256 << 20, dtype=torch.uint8, device=dev)
    copies = [[qlin.quantize((torch.randn(*shapes[w], generator=g, device=dev) * 0.02).half(),
                             bits, 64) for w in mats] for _ in range(4)]
    k = shapes[mats[0]][1]
    X = torch.randn(m, k, generator=g, device=dev).half()
    Ys = [torch.empty(m, shapes[w][0], device=dev) for w in mats]
    h16 = torch.empty(m, shapes[mats[0]][0], dtype=torch.float16, device=dev)
    qlin.set_launch_override('gemm', None if form == 'default' else form)
    for it in range(8):
        c = copies[it % 4]
        if case == 'qkv':
            qlin.gemm_multi(c, X, Ys, ws=ws)
        elif case == 'pair':
            qlin.gemm_swiglu(c[0], c[1], X, None, h16, ws=ws, want_h=False)
        else:
            qlin.gemm(c[0], X, Ys[0], ws=ws)
    torch.cuda.synchronize()
    qlin.set_launch_override('gemm', None)
    print("done", argv[0], case, form, bits, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
