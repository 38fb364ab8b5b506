"""GPU parity of qlin_quantize_batch (a lever move: every master re-quantized
in as few launches as possible): scales, zeros and packed words bit-exact
against the oracle, identical to one qlin_quantize per matrix, for mixed
shapes, with and without codes, and across the 64-job launch boundary."""
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


SHAPES = [(200, 192), (64, 64), (1, 128), (130, 896), (896, 896), (128, 4864), (300, 320)]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("group", [64, "K"])
@pytest.mark.parametrize("codes", [True, False])
def test_quantize_batch_matches_oracle(bits, group, codes):
    rng = np.random.default_rng([91, bits, 0 if group == "K" else 1, int(codes)])
    masters = [synth.master_weights(rng, n, k) if i % 2 else synth.edge_groups(bits, rng, n, k)
               for i, (n, k) in enumerate(SHAPES)]
    say(f"quantize batch bits={bits} group={group} codes={codes}")
    outs = qlin.quantize_batch([dev(w) for w in masters], bits, group, codes=codes)
    torch.cuda.synchronize()
    for w16, q in zip(masters, outs):
        n, k = w16.shape
        g = k if group == "K" else 64
        c, s16, z = oracle.quantize(w16, bits, g)
        assert np.array_equal(q.scale.cpu().numpy().view(np.uint16)[:oracle.tile_meta(s16).size],
                              oracle.tile_meta(s16).view(np.uint16)), (n, k)
        assert np.array_equal(q.zero.cpu().numpy()[:oracle.tile_meta(z).size], oracle.tile_meta(z))
        if codes:
            assert np.array_equal(q.data.cpu().numpy().view(np.uint32), oracle.pack_codes(c, bits))


def test_quantize_batch_many_jobs_equals_single_calls():
    """70 matrices (two launches of 64 + 6) give exactly what 70 single calls give."""
    rng = np.random.default_rng(92)
    shapes = [(int(rng.integers(1, 300)), 64 * int(rng.integers(1, 20))) for _ in range(70)]
    masters = [dev(synth.master_weights(rng, n, k)) for n, k in shapes]
    for bits, group in ((4, 64), (3, "K")):
        say(f"quantize batch of 70, bits={bits} group={group}")
        batch = qlin.quantize_batch(masters, bits, group)
        single = [qlin.quantize(w, bits, group) for w in masters]
        torch.cuda.synchronize()
        for a, b in zip(batch, single):
            assert torch.equal(a.data, b.data)
            assert torch.equal(a.scale.view(torch.int16), b.scale.view(torch.int16))
            assert torch.equal(a.zero, b.zero)
    # re-quantizing into the same buffers at another bit width (the lever moving)
    outs = qlin.quantize_batch(masters, 2, 64, codes=False)
    again = qlin.quantize_batch(masters, 8, 64, codes=False, outs=outs)
    torch.cuda.synchronize()
    for w, o in zip(masters, again):
        _, s16, z = oracle.quantize(w.cpu().numpy(), 8, 64)
        assert np.array_equal(o.scale.cpu().numpy().view(np.uint16)[:oracle.tile_meta(s16).size],
                              oracle.tile_meta(s16).view(np.uint16))
