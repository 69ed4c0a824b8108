"""Seeded synthetic inputs for the fused quantize -> int8 GEMM -> dequant linear layer.

This module only draws random numbers. It holds none of the method's arithmetic
(no scales, no rounding to int8, no products), so both the CPU oracle and the
GPU path can take their inputs from here without sharing any computation.

Recipe (one generator per (workload, shape), numpy PCG64, seed 0 unless given):

1. ``W = standard_normal((N, K), float32) * 0.02`` -- weights ~ N(0, 0.02^2).
2. ``idx = choice(K, n_out, replace=False)`` with ``n_out = floor(0.01*K + 0.5)``:
   the 1 % of input channels that carry activation outliers.
3. ``x = standard_normal((M, K), float32)``; ``x[:, idx] *= 50``; ``x -> float16``.

Because W and idx are drawn before x, they do not depend on M, and the rows of
x are prefix-consistent across an M sweep (the first M rows of a larger draw).

The pages measure on models (Qwen3, Llama3) and on Wikitext2 perplexity; none of
that is available here, so these seeded tensors stand in for one linear layer's
weights and for prefill activations with a few outlier channels (the outlier
behaviour the pages describe for LLM activations).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "n_outlier_channels",
    "linear_inputs",
    "qwen3_8b_block_inputs",
    "rmsnorm_inputs",
    "QWEN3_8B_BLOCK",
]


def n_outlier_channels(K: int) -> int:
    """Number of outlier input channels: floor(0.01*K + 0.5)."""
    return int(np.floor(0.01 * K + 0.5))


def _draw_weight(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    return rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)


def _draw_activation(rng: np.random.Generator, M: int, K: int, idx: np.ndarray) -> np.ndarray:
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[:, idx] *= np.float32(50.0)
    return x.astype(np.float16)


def linear_inputs(M: int, N: int, K: int, seed: int = 0):
    """Weights W fp32 [N, K] and activations x fp16 [M, K] for one linear layer.

    Returns ``(x, W)`` as numpy arrays. M may be 0 (an empty activation batch).
    """
    rng = np.random.default_rng(seed)
    W = _draw_weight(rng, N, K)
    idx = rng.choice(K, n_outlier_channels(K), replace=False)
    x = _draw_activation(rng, M, K, idx)
    return x, W


# One Qwen3-8B-shaped decoder block: (name, in_features K, out_features N).
QWEN3_8B_BLOCK = (
    ("q", 4096, 4096),
    ("k", 4096, 1024),
    ("v", 4096, 1024),
    ("o", 4096, 4096),
    ("gate", 4096, 12288),
    ("up", 4096, 12288),
    ("down", 12288, 4096),
)

# Which block input feeds which projection.
QWEN3_8B_BLOCK_INPUTS = (
    ("attn_in", 4096, ("q", "k", "v")),
    ("o_in", 4096, ("o",)),
    ("mlp_in", 4096, ("gate", "up")),
    ("down_in", 12288, ("down",)),
)


def qwen3_8b_block_inputs(M: int = 2048, seed: int = 0):
    """Seven weights (q, k, v, o, gate, up, down) then four block inputs.

    Returns ``(inputs, weights)``: dicts name -> numpy array. Weights are drawn
    first in projection order, then each input with its own outlier channels
    (the activation distribution of the single-linear workload).
    """
    rng = np.random.default_rng(seed)
    weights = {name: _draw_weight(rng, N, K) for name, K, N in QWEN3_8B_BLOCK}
    inputs = {}
    for name, K, _ in QWEN3_8B_BLOCK_INPUTS:
        idx = rng.choice(K, n_outlier_channels(K), replace=False)
        inputs[name] = _draw_activation(rng, M, K, idx)
    return inputs, weights


def rmsnorm_inputs(M: int, K: int, seed: int = 0):
    """Input rows and a norm weight for the RMSNorm producer of a linear layer's input.

    ``x`` [M, K] fp16 as in ``linear_inputs`` (standard normal, 1 % outlier channels x 50),
    drawn after ``idx``; then ``g = 1 + 0.1 * standard_normal(K)`` as fp16 -- a norm weight
    near one, spread like a trained one. (No trained weights are available; these stand in.)
    """
    rng = np.random.default_rng(seed)
    idx = rng.choice(K, n_outlier_channels(K), replace=False)
    x = _draw_activation(rng, M, K, idx)
    g = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float16)
    return x, g
