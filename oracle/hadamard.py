"""16-point random Hadamard transform (RHT) of the weight-gradient inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: gist.science, "Pretraining Large Language Models with NVFP4",
Resumen técnico §2 "Transformadas de Hadamard Aleatorias (RHT)" -- a random
orthogonal transform is applied to the inputs of the weight-gradient GEMM to
spread outliers toward a Gaussian shape, with a 16x16 Hadamard matrix and one
random sign vector that stays fixed for the whole run; news.hamidun.com,
"NVIDIA desarrolló un método ...", "Cómo Funciona" (16x16 random Hadamard
transforms of the gradient inputs).

Readings:

* H is the Sylvester Hadamard matrix in natural order,
  ``H[i][j] = (-1)^popcount(i & j)``.
* The transform of 16 consecutive values x (16 consecutive tokens of one
  column, the contraction dimension of the weight-gradient GEMM) is
  ``x' = (1/4) * H @ (d * x)``: orthonormal, so the same transform on both
  operands cancels in dY^T X.
* The sign vector d comes from the seed: ``d_i = 1 - 2 * bit_i(W0)`` where W0
  is the first word of Philox4x32-10 with key (seed low, seed high) and
  counter (0, 0, 0, 2).
* The oracle computes the product exactly in float64 and rounds once to
  float32.
"""

from __future__ import annotations

import numpy as np

from .philox import STREAM_RHT_SIGNS, philox4x32_10


def hadamard16() -> np.ndarray:
    """16x16 Sylvester Hadamard matrix (int64) from the popcount definition."""
    i = np.arange(16)[:, None]
    j = np.arange(16)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def rht_signs(seed: int) -> np.ndarray:
    """The 16 signs (+1 / -1, int64) of the fixed random diagonal."""
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w0 = int(philox4x32_10(key, np.array([0, 0, 0, STREAM_RHT_SIGNS], dtype=np.uint64))[0])
    bits = np.array([(w0 >> i) & 1 for i in range(16)], dtype=np.int64)
    return 1 - 2 * bits


def rht(x, seed: int) -> np.ndarray:
    """RHT along axis 0 (tokens) of a [T, C] matrix, in blocks of 16 tokens.

    Returns float32 [T, C]; T must be a multiple of 16.
    """
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[0] % 16 != 0:
        raise ValueError("rht expects [T, C] with T % 16 == 0")
    t, c = x.shape
    m = hadamard16().astype(np.float64) * rht_signs(seed)[None, :].astype(np.float64) / 4.0
    blocks = x.astype(np.float64).reshape(t // 16, 16, c)
    out = np.matmul(m[None, :, :], blocks)  # [T/16, 16, C]
    return out.reshape(t, c).astype(np.float32)
