"""The decode step's algorithmic bytes (the numerator of bench.py's headline
GB/s and of its roofline figure), recounted from the Qwen2.5-0.5B shapes.

Per packed int4 g64 weight: n*k/2 code bytes + n*k/64 fp16 scales (2 B) +
n*k/64 uint8 zeros.  Per launch of the step: the fp16 x it reads and the
outputs it writes (fp32 y; fp16 h for the gate/up pair, read back by down).
"""
import bench
import synth


class _NoLaunch:
    """Stands in for the binding: the step's launch functions are built,
    never called."""
    def __getattr__(self, name):
        raise AssertionError(f"qlin.{name} called while counting bytes")


def recount():
    shapes = synth.qwen25_decode_shapes()
    hidden, inter, kv = 896, 4864, 128
    vocab = 151936
    weights = sum(n * k // 2 + 3 * n * k // 64 for (_, _, n, k) in shapes)
    per_layer = (2 * hidden + 4 * (hidden + 2 * kv)      # q/k/v set: x, three y
                 + 2 * hidden + 4 * hidden               # o
                 + 2 * hidden + 2 * inter                # gate/up: x, fp16 h
                 + 2 * inter + 4 * hidden)               # down: h, y
    layers = len({l for (l, nm, _, _) in shapes if nm != "lm_head"})
    return weights + layers * per_layer + 2 * hidden + 4 * vocab


def test_wbytes_int4_g64():
    assert bench.wbytes(896, 4864, 4, 64) == 896 * 4864 // 2 + 896 * 76 * 3
    assert bench.wbytes(64, 128, 3, "row") == 64 * 128 * 3 // 8 + 64 * 3


def test_decode_step_bytes_and_launches():
    import torch
    shapes = synth.qwen25_decode_shapes()
    assert len(shapes) == 169
    xs = [torch.empty(k, dtype=torch.float16) for (_, _, _, k) in shapes]
    calls, nbytes, launches = bench.grouped_step_calls(_NoLaunch(), shapes, [None] * len(shapes),
                                                       xs, "cpu", torch, None)
    assert launches == len(calls) == 24 * 4 + 1
    assert nbytes == recount() == 271_623_168
