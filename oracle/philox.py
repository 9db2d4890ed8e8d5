"""Philox4x32-10 counter-based generator and the stochastic-rounding bit map.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages only say that gradients are rounded at random ("tira un dado" in
gist.science, "Pretraining Large Language Models with NVFP4", Lo esencial,
item 4; Resumen técnico §2 "Escalado Bidimensional (2D) y Redondeo
Estocástico"). They name no generator. The generator is Philox4x32 with ten
rounds, from its published definition: J. K. Salmon, M. A. Moraes,
R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
SC'11. A round multiplies two of the four 32-bit counter words by fixed odd
constants, keeps both halves of each 64-bit product, and mixes the high
halves with the other two words and the two key words by xor; the key is
advanced by two Weyl constants between rounds.

Reading of how the bits are used (the pages say nothing):

* key = (seed low 32 bits, seed high 32 bits);
* one call serves 8 consecutive elements of the quantized tensor, counted in
  the orientation that is stored: element ``e`` (row-major linear index of the
  stored matrix) uses group ``g = e >> 3`` and counter
  ``(g low, g high, offset, stream)``;
* ``stream`` is 0 for a row-blocked copy, 1 for a column-blocked (transposed)
  copy, 2 for the Hadamard sign vector;
* element ``e`` takes the 16-bit half ``e & 1`` (0 = low) of word ``(e & 7) >> 1``.
"""

from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)

STREAM_ROW = 0
STREAM_COL = 1
STREAM_RHT_SIGNS = 2


def philox4x32_10(key, counter) -> np.ndarray:
    """Philox4x32-10 of each counter.

    key: pair of uint32 (k0, k1).
    counter: array [..., 4] of uint32 words (c0, c1, c2, c3).
    Returns uint32 array [..., 4].
    """
    c = np.asarray(counter, dtype=np.uint64)
    if c.shape[-1] != 4:
        raise ValueError("counter must have 4 words")
    x0, x1, x2, x3 = (c[..., i] & _MASK32 for i in range(4))
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = m0 * x0  # < 2^64, exact in uint64
        p1 = m1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def sr_random_u16(seed: int, offset: int, stream: int, e) -> np.ndarray:
    """16-bit random integer that stochastic rounding of element ``e`` uses.

    e: array of element linear indices (int64) in the stored orientation.
    """
    e = np.asarray(e, dtype=np.int64)
    g = (e >> 3).astype(np.uint64)
    ctr = np.stack(
        [
            g & _MASK32,
            g >> np.uint64(32),
            np.full_like(g, offset & 0xFFFFFFFF),
            np.full_like(g, stream & 0xFFFFFFFF),
        ],
        axis=-1,
    )
    words = philox4x32_10((seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF), ctr)
    w = np.take_along_axis(words, ((e & 7) >> 1)[..., None], axis=-1)[..., 0]
    return ((w.astype(np.uint32) >> ((e & 1) * 16).astype(np.uint32)) & 0xFFFF).astype(np.uint16)
