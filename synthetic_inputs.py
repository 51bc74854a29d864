"""Seeded synthetic inputs for the quantized DiT linear layer.

The pages evaluate on audio produced from trained Stable Audio 3 weights, which
are not available; these seeded normal tensors stand in for the diffusion
transformer's weights and activations at its real shapes.  This module holds no
step of the method (no quantization, packing, contraction or epilogue): it only
draws numbers, so both the HIP path's tests/benchmark and the CPU oracle can
consume the very same inputs.

Recipe: ``numpy.random.default_rng(seed).standard_normal(shape, float32) * sigma``
then ``.astype(float16)`` (round to nearest even).  The steering direction is
drawn in fp64, divided by its fp64 2-norm and stored as fp32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# width of the DiT at the small-music scale used for the single-layer workloads
WIDTH = 1536
MLP = 6144
TOKENS = 2048  # 2 classifier-free-guidance branches x 1024 latent tokens


def normal_f16(shape, sigma: float, seed: int, offset: float = 0.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    if offset:
        v = v + np.float32(offset)
    return v.astype(np.float16)


def unit_direction(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    d = rng.standard_normal(n)  # fp64
    return (d / np.sqrt(np.sum(d * d))).astype(np.float32)


@dataclass
class Linear:
    """One linear's inputs: X fp16 [M][K], W fp16 [K][N] (+ optional bias fp16 [N])."""
    name: str
    x: np.ndarray
    w: np.ndarray
    bias: np.ndarray | None = None
    gelu: bool = False


def small_w8a8() -> Linear:
    """Single W8A8 linear: X[64x256], W[256x256], both N(0,1)."""
    return Linear("w8a8_64x256x256", normal_f16((64, 256), 1.0, 101), normal_f16((256, 256), 1.0, 102))


def mlp_up_w8a16() -> Linear:
    """W8A16 MLP-up at DiT width: X[2048x1536] N(0,1), W[1536x6144] N(0,0.02),
    bias[6144] N(0,0.01), GELU(tanh)."""
    return Linear("w8a16_2048x1536x6144", normal_f16((TOKENS, WIDTH), 1.0, 201),
                  normal_f16((WIDTH, MLP), 0.02, 202), normal_f16((MLP,), 0.01, 203), True)


def w4a16_sweep_x() -> np.ndarray:
    """One [2048x1536] N(0,1) draw; the M-point of the sweep takes its first M rows."""
    return normal_f16((TOKENS, WIDTH), 1.0, 301)


def w4a16_w() -> np.ndarray:
    return normal_f16((WIDTH, MLP), 0.02, 302)


W4A16_M_SWEEP = (16, 256, 2048)


def dit_block() -> dict:
    """W8A8 DiT block chain at M=2048, width 1536: h, the four weights, d, alpha."""
    return {
        "h": normal_f16((TOKENS, WIDTH), 1.0, 401),
        "qkv": normal_f16((WIDTH, 3 * WIDTH), 0.02, 402),
        "o": normal_f16((WIDTH, WIDTH), 0.02, 403),
        "up": normal_f16((WIDTH, MLP), 0.02, 404),
        "down": normal_f16((MLP, WIDTH), 0.02, 405),
        "d": unit_direction(WIDTH, 406),
        "alpha": 0.3,
    }


HEADS = 24      # 64-dimensional attention heads at width 1536
SEQ = 1024      # latent tokens per guidance branch


def dit_block_norms() -> dict:
    """LayerNorm parameters of the full block: gamma ~ 1 + N(0, 0.1), beta ~ N(0, 0.1)."""
    return {
        "ln1": (normal_f16((WIDTH,), 0.1, 407, offset=1.0), normal_f16((WIDTH,), 0.1, 408)),
        "ln2": (normal_f16((WIDTH,), 0.1, 409, offset=1.0), normal_f16((WIDTH,), 0.1, 410)),
    }


# 1.2B-parameter-scale denoising step: 24 blocks at width 2048, MLP 8192
STEP_BLOCKS = 24
STEP_WIDTH = 2048
STEP_MLP = 8192
STEP_LAYERS = (("qkv", STEP_WIDTH, 3 * STEP_WIDTH), ("o", STEP_WIDTH, STEP_WIDTH),
               ("up", STEP_WIDTH, STEP_MLP), ("down", STEP_MLP, STEP_WIDTH))


def step_weight(block: int, layer: int) -> np.ndarray:
    _, k, n = STEP_LAYERS[layer]
    return normal_f16((k, n), 0.02, 5000 + 10 * block + layer)


def step_x(k: int) -> np.ndarray:
    """Input shared by every linear of the step with this K (2048 or 8192)."""
    return normal_f16((TOKENS, k), 1.0, 501 if k == STEP_WIDTH else 502)
