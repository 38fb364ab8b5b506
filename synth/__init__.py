"""Seeded synthetic inputs and the linear-layer shapes of the measured models.

Shared by the tests, the bench and the smoke check.  Holds no arithmetic of
the method (no quantization, no matmul): only random draws and shape tables,
so both the oracle side and the HIP side can take their inputs from here.

The pages run real checkpoints (Qwen2.5-0.5B-Instruct on the Enargeia page,
Qwen3-0.6B in Bitcrush, Qwen3-8B in Trellis-WebGPU).  Their weights are not
available, so every matrix here has the real linear-layer shape and synthetic
values: weights ~ N(0, 0.02) drawn in binary32 and rounded to fp16 (the fp16
master), activations ~ N(0, 1) in fp16.
"""
from __future__ import annotations

import numpy as np

WEIGHT_STD = np.float32(0.02)

# (name, N = out features, K = in features) per transformer layer.
QWEN25_05B_LAYER = (
    ("q", 896, 896), ("k", 128, 896), ("v", 128, 896), ("o", 896, 896),
    ("gate", 4864, 896), ("up", 4864, 896), ("down", 896, 4864),
)
QWEN25_05B_LAYERS = 24
QWEN25_05B_LM_HEAD = ("lm_head", 151936, 896)   # tied to the embedding
QWEN25_05B_EXTRA_PARAMS = 27648 + 43904          # q/k/v biases + norm weights

QWEN3_06B_LAYER = (
    ("q", 2048, 1024), ("k", 1024, 1024), ("v", 1024, 1024), ("o", 1024, 2048),
    ("gate", 3072, 1024), ("up", 3072, 1024), ("down", 1024, 3072),
)
QWEN3_06B_LAYERS = 28
QWEN3_06B_EMBED = (151936, 1024)
QWEN3_06B_NORM_PARAMS = 65536

QWEN3_8B_LAYER = (
    ("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
    ("gate", 12288, 4096), ("up", 12288, 4096), ("down", 4096, 12288),
)
QWEN3_8B_LAYERS = 36

MAT_INDEX = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6,
             "lm_head": 7}


def master_weights(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """fp16 [n, k] master weights: binary32 N(0, 0.02) draws rounded to fp16."""
    return (rng.standard_normal((n, k), dtype=np.float32) * WEIGHT_STD).astype(np.float16)


def activations(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    """fp16 [m, k] activations from binary32 N(0, 1) draws."""
    return rng.standard_normal((m, k), dtype=np.float32).astype(np.float16)


def single_gemv_case(seed: int = 0):
    """The 896x896 int4 g64 decode GEMV case: W drawn first, then x."""
    rng = np.random.default_rng(seed)
    w = master_weights(rng, 896, 896)
    x = activations(rng, 1, 896)[0]
    return w, x


def layer_rng(cfg: int, layer: int, mat: str) -> np.random.Generator:
    return np.random.default_rng([cfg, layer, MAT_INDEX[mat]])


def act_rng(cfg: int, layer: int, mat: str) -> np.random.Generator:
    return np.random.default_rng([cfg, 1000 + layer, MAT_INDEX[mat]])


def qwen25_decode_shapes(include_lm_head: bool = True):
    """[(layer, name, N, K)] of one Qwen2.5-0.5B decode step (169 matrices)."""
    out = [(l, nm, n, k) for l in range(QWEN25_05B_LAYERS) for nm, n, k in QWEN25_05B_LAYER]
    if include_lm_head:
        nm, n, k = QWEN25_05B_LM_HEAD
        out.append((QWEN25_05B_LAYERS, nm, n, k))
    return out


def qwen3_06b_shapes():
    return [(l, nm, n, k) for l in range(QWEN3_06B_LAYERS) for nm, n, k in QWEN3_06B_LAYER]


def qwen3_8b_shapes():
    return [(l, nm, n, k) for l in range(QWEN3_8B_LAYERS) for nm, n, k in QWEN3_8B_LAYER]


def edge_groups(bits: int, rng: np.random.Generator, n_rows: int = 64, k: int = 256) -> np.ndarray:
    """fp16 [n_rows, k] masters whose 64-groups hit the quantizer's special
    cases: constant groups, one-signed groups, exact half-way ties, extremes
    that clamp, tiny and huge magnitudes, signed zeros, subnormals."""
    w = master_weights(rng, n_rows, k).astype(np.float32)
    g = w.reshape(n_rows, k // 64, 64)
    kinds = rng.integers(0, 8, size=(n_rows, k // 64))
    for r in range(n_rows):
        for j in range(k // 64):
            kind = kinds[r, j]
            if kind == 0:      # constant group
                g[r, j, :] = np.float32(rng.standard_normal()) * np.float32(0.05)
            elif kind == 1:    # one-signed, away from zero
                g[r, j, :] = np.float32(1.0) + np.abs(g[r, j, :])
            elif kind == 2:    # dyadic grid -> many exact ties
                qm = (1 << bits) - 1
                step = np.float32(2.0 ** -6)
                ints = rng.integers(0, 2 * qm + 1, size=64).astype(np.float32)
                g[r, j, :] = (ints - np.float32(qm)) * step / np.float32(2)
                g[r, j, 0] = -np.float32(qm) * step / np.float32(2)
                g[r, j, 1] = np.float32(qm) * step / np.float32(2)
            elif kind == 3:    # two extremes, rest zero (clamps at the top)
                g[r, j, :] = 0
                g[r, j, 0], g[r, j, 1] = -1.0, 1.0
            elif kind == 4:    # tiny magnitudes incl. subnormals and -0
                g[r, j, :] = g[r, j, :] * np.float32(1e-4)
                g[r, j, 3] = -0.0
            elif kind == 5:    # large magnitudes
                g[r, j, :] = g[r, j, :] * np.float32(1e5)
            elif kind == 6:    # negative one-signed
                g[r, j, :] = -np.float32(2.0) - np.abs(g[r, j, :])
            # kind 7: plain random
    out = g.reshape(n_rows, k)
    return np.clip(out, -60000, 60000).astype(np.float16)
