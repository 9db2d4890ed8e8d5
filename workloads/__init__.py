"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and rounds them to the input dtype; it
holds none of the NVFP4 arithmetic, so both the GPU library's tests and the
oracle can take their inputs from it without sharing any of the method.

The pages describe a 12B hybrid Mamba-Transformer trained on 10T tokens
(gist.science, "Pretraining Large Language Models with NVFP4", Resumen
técnico §3-4; deultimominuto.info, "NVFP4 en la práctica"); no layer shapes,
weights or data are given or available. These tensors stand in for that
model's linear-layer operands: activations N(0, 1) with a few outlier
channels, weights N(0, 0.02^2), gradients Laplace(0, 1e-3).

Every generator returns a C-contiguous float32 numpy array. ``dtype="bf16"``
rounds the values to bfloat16 (round to nearest even, through torch's CPU
cast) and keeps them as float32, so the bytes handed to the GPU as bfloat16
and the values the oracle sees are the same numbers.
"""

from __future__ import annotations

import numpy as np


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and return them as float32."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_values(x)
    if dtype == "fp32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(shape, seed: int, std: float = 1.0, outlier_channels: int = 0,
           channel_gain: float = 20.0, outlier_fraction: float = 0.0,
           element_gain: float = 50.0, dtype: str = "bf16") -> np.ndarray:
    """std * N(0, 1) of ``shape`` [rows, cols].

    outlier_channels: that many columns (drawn without replacement from the
    same generator) are multiplied by ``channel_gain``.
    outlier_fraction: round(fraction * size) entries (distinct flat indices
    from the same generator) are multiplied by ``element_gain``.
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if outlier_channels:
        ch = rng.choice(shape[1], outlier_channels, replace=False)
        x[:, ch] *= np.float32(channel_gain)
    if outlier_fraction:
        n = int(round(outlier_fraction * x.size))
        idx = rng.choice(x.size, n, replace=False)
        x.reshape(-1)[idx] *= np.float32(element_gain)
    return _finish(x, dtype)


def laplace(shape, seed: int, b: float = 1e-3, dtype: str = "bf16") -> np.ndarray:
    """Laplace(0, b) of ``shape``."""
    rng = np.random.default_rng(seed)
    return _finish(rng.laplace(0.0, b, shape).astype(np.float32), dtype)


# ---------------------------------------------------------------------------
# The five workloads (tensor shapes of one linear layer of the 12B model:
# hidden 5120, FFN 20480; 8192 or 16384 tokens).
# ---------------------------------------------------------------------------

RHT_SEED = 7
SR_SEED = 7


def fp32_outlier_matrix():
    """fp32 256x1024, N(0,1), 0.1% of entries x50, seed 0 (1x16 RN round trip)."""
    return normal((256, 1024), seed=0, outlier_fraction=0.001, element_gain=50.0, dtype="fp32")


def activation(tokens: int = 8192, hidden: int = 5120, seed: int = 1):
    """bf16 activations, N(0,1) with 16 outlier channels x20."""
    return normal((tokens, hidden), seed=seed, outlier_channels=16, channel_gain=20.0)


def weight(rows: int = 20480, cols: int = 5120, seed: int = 2):
    """bf16 weight, N(0, 0.02^2)."""
    return normal((rows, cols), seed=seed, std=0.02)


def gradient(tokens: int = 8192, cols: int = 20480, seed: int = 3):
    """bf16 output gradient dY, Laplace(0, 1e-3)."""
    return laplace((tokens, cols), seed=seed, b=1e-3)


def wgrad_activation(tokens: int = 8192, hidden: int = 5120, seed: int = 4):
    """bf16 activation X for the weight-gradient path, N(0,1)."""
    return normal((tokens, hidden), seed=seed)


def linear_layer(tokens: int = 16384, hidden: int = 5120, ffn: int = 20480):
    """X [tokens, hidden] (seed 5, 16 outlier channels), W [ffn, hidden]
    (seed 2), dY [tokens, ffn] (seed 6)."""
    x = normal((tokens, hidden), seed=5, outlier_channels=16, channel_gain=20.0)
    w = weight(ffn, hidden, seed=2)
    dy = laplace((tokens, ffn), seed=6, b=1e-3)
    return x, w, dy
