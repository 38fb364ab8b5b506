"""Oracle vs the hand-worked one-group examples in tests/golden/.

The fixtures were worked out by hand (see tests/golden/README.md for the
sources): they pin the scale, zero point, code and dequantized-weight
arithmetic, including ties (round half to even), the fp16 scale rounding
down into a clamp, the constant-group guard and every supported bit width.
"""
import glob
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _expand(tokens, cast):
    out = []
    for t in tokens:
        if "*" in t:
            v, n = t.split("*")
            out.extend([cast(v)] * int(n))
        else:
            out.append(cast(t))
    return out


def load_example(path):
    d = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(":", 1)
            d[key.strip()] = val.split()
    return {
        "bits": int(d["bits"][0]),
        "group": int(d["group"][0]),
        "w": np.array(_expand(d["w"], float), dtype=np.float64),
        "scale16": int(d["scale16"][0], 16),
        "zero": int(d["zero"][0]),
        "codes": np.array(_expand(d["codes"], int), dtype=np.int64),
        "what": np.array(_expand(d["what"], float), dtype=np.float64),
    }


EXAMPLES = sorted(glob.glob(os.path.join(GOLDEN, "example_*.txt")))


def test_fixtures_present():
    assert len(EXAMPLES) >= 7


@pytest.mark.parametrize("path", EXAMPLES, ids=[os.path.basename(p) for p in EXAMPLES])
def test_worked_example(path):
    ex = load_example(path)
    w64 = ex["w"]
    assert w64.size == 64
    w16 = w64.astype(np.float16)
    assert np.array_equal(w16.astype(np.float64), w64), "fixture weights must be fp16-exact"
    w16 = w16.reshape(1, 64)
    codes, s16, z = oracle.quantize(w16, ex["bits"], ex["group"])
    assert int(s16.view(np.uint16)[0, 0]) == ex["scale16"]
    assert int(z[0, 0]) == ex["zero"]
    assert np.array_equal(codes[0].astype(np.int64), ex["codes"])
    what = oracle.dequantize(codes, s16, z, ex["group"])
    assert np.array_equal(what[0], ex["what"])


@pytest.mark.parametrize("path", EXAMPLES, ids=[os.path.basename(p) for p in EXAMPLES])
def test_worked_example_permuted_and_tiled(path):
    """The group's result does not depend on where in the group, or in which
    row of a multi-row matrix, the values sit."""
    ex = load_example(path)
    rng = np.random.default_rng(7)
    perm = rng.permutation(64)
    w16 = ex["w"].astype(np.float16)[perm]
    mat = np.zeros((3, 128), dtype=np.float16)
    mat[1, 64:] = w16
    mat[0, :64] = np.float16(1)          # a constant group elsewhere
    mat[2, :] = np.linspace(-1, 1, 128).astype(np.float16)
    codes, s16, z = oracle.quantize(mat, ex["bits"], 64)
    assert int(s16.view(np.uint16)[1, 1]) == ex["scale16"]
    assert int(z[1, 1]) == ex["zero"]
    assert np.array_equal(codes[1, 64:].astype(np.int64), ex["codes"][perm])


def test_one_signed_group_clamps_zero_point():
    """64 values evenly spaced on [1.0, 1.1], 4-bit: the zero point
    rint(-1.0 / s) is far below 0 and clamps to 0, every code saturates at 15
    and the error is about 150 scales (no widening of the range to include 0)."""
    w16 = np.linspace(1.0, 1.1, 64).astype(np.float16).reshape(1, 64)
    codes, s16, z = oracle.quantize(w16, 4, 64)
    # d = fp16(1.1) - 1 = 0.099609375; /15 = 0.006640625; fp16 step 2^-18
    # -> 1740.8 -> 1741 * 2^-18 = 0.006641387939453125
    assert float(s16[0, 0]) == 0.006641387939453125
    assert int(z[0, 0]) == 0
    assert np.all(codes == 15)
    err = np.abs(w16.astype(np.float64) - oracle.dequantize(codes, s16, z, 64))
    assert 150 < err.max() / float(s16[0, 0]) < 151
