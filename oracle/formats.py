"""Element and scale formats of NVFP4, written from their bit-field definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: gist.science, "Pretraining Large Language Models with NVFP4",
Resumen técnico §2 "Formato NVFP4" (4-bit elements in 16-element blocks, an
E4M3 block scale with 4 exponent and 3 mantissa bits, an FP32 tensor scale);
deultimominuto.info, "Cómo funciona NVFP4" (a 4-bit element takes only 16
distinct values).

Readings (the pages fix none of these):

* E2M1 element: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; no
  infinities or NaN. Code ``q = sign<<3 | exp<<1 | man``. Magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6} for codes 0..7; codes 8..15 are their
  negatives, so +0 and -0 are both codes and "16 distinct values" counts them
  separately.
* E4M3 scale: the E4M3FN variant -- bias 7, no infinities, 0x7F and 0xFF are
  NaN, largest finite value 448 (0x7E), subnormals m * 2^-9.
* Rounding to E2M1 (RN): nearest magnitude; a value exactly half way between
  two magnitudes goes to the code whose mantissa bit is 0; anything above 6
  becomes 6 (saturation). The sign bit of the code is the sign bit of the
  input, so a negative value that rounds to zero gives code 0x8.
* Rounding to E4M3 (block scale): nearest finite value, ties to even mantissa,
  saturating at 448 -- never NaN.
* Stochastic rounding to E2M1: with ``a = min(|y|, 6)``, ``lo`` the largest
  magnitude <= a and ``hi`` the next one, round up to ``hi`` exactly when
  ``(a - lo) / (hi - lo) + u16 / 2^16 >= 1``, with ``u16`` a uniform 16-bit
  random integer: the random fraction is added below the grid step and the
  sum is truncated, which rounds up with probability floor(frac * 2^16) /
  2^16. The pages only say that gradients are rounded at random so that the
  rounding is unbiased (Resumen técnico §2, "Escalado Bidimensional (2D) y
  Redondeo Estocástico"; Lo esencial, item 4).
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# E2M1
# --------------------------------------------------------------------------


def _e2m1_magnitude_from_bits(code: int) -> float:
    """Magnitude of a 3-bit E2M1 magnitude code, from the bit fields."""
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return 0.5 * m  # subnormal: 2^(1-bias) * (m / 2) with bias 1
    return float(2.0 ** (e - 1) * (1.0 + m / 2.0))


#: The 8 non-negative E2M1 magnitudes, indexed by the 3-bit magnitude code.
E2M1_MAGNITUDES = np.array([_e2m1_magnitude_from_bits(c) for c in range(8)], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit code (array of ints 0..15) as float64."""
    codes = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[codes & 0x7]
    return np.where((codes & 0x8) != 0, -mag, mag)


def e2m1_encode_rn(y) -> np.ndarray:
    """Round-to-nearest-even E2M1 code (uint8, 0..15) of each float32 ``y``.

    Definition: the code whose magnitude is nearest to |y| (ties to the code
    with mantissa bit 0, values above 6 saturate to 6), carrying y's sign bit.
    ``y`` must be finite.
    """
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("e2m1_encode_rn: non-finite input")
    a = np.abs(y).astype(np.float64)  # exact
    mags = E2M1_MAGNITUDES
    # hi = index of the first magnitude >= a (clipped to the last one)
    hi = np.searchsorted(mags, a, side="left")
    hi = np.minimum(hi, 7)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    # above 6: d_hi < 0 -> nearest is 6 (hi == 7)
    pick_hi = np.where(d_hi < d_lo, True, np.where(d_hi > d_lo, False, (hi & 1) == 0))
    pick_hi = np.where(hi == lo, True, pick_hi)
    mag_code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 3
    return (mag_code | sign).astype(np.uint8)


def e2m1_encode_sr(y, u16) -> np.ndarray:
    """Stochastically rounded E2M1 code of each float32 ``y`` given 16-bit
    random integers ``u16`` (same shape). See the module docstring."""
    y = np.asarray(y, dtype=np.float32)
    u16 = np.asarray(u16).astype(np.int64)
    if not np.all(np.isfinite(y)):
        raise ValueError("e2m1_encode_sr: non-finite input")
    if y.shape != u16.shape:
        raise ValueError("e2m1_encode_sr: shape mismatch")
    mags = E2M1_MAGNITUDES
    a = np.minimum(np.abs(y).astype(np.float64), mags[7])
    lo = np.searchsorted(mags, a, side="right") - 1  # mags[lo] <= a
    hi = np.minimum(lo + 1, 7)
    step = mags[hi] - mags[lo]
    frac = np.where(step > 0, (a - mags[lo]) / np.where(step > 0, step, 1.0), 0.0)
    # frac + u16 / 2^16 >= 1, compared exactly: frac * 2^16 is exact in
    # float64 (a power-of-two scaling) and 2^16 - u16 is an integer
    mag_code = np.where(frac * 65536.0 >= 65536 - u16, hi, lo).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 3
    return (mag_code | sign).astype(np.uint8)


# --------------------------------------------------------------------------
# E4M3 (FN variant)
# --------------------------------------------------------------------------


def _e4m3_value_from_bits(byte: int) -> float:
    """Value of an E4M3FN byte, from the bit fields (NaN for 0x7F / 0xFF)."""
    s = (byte >> 7) & 0x1
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        v = 2.0 ** (1 - 7) * (m / 8.0)
    else:
        v = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -v if s else v


_E4M3_TABLE = np.array([_e4m3_value_from_bits(b) for b in range(256)], dtype=np.float64)
# Non-negative finite values, bytes 0x00..0x7E, strictly increasing.
_E4M3_POS = _E4M3_TABLE[:0x7F].copy()
E4M3_MAX = float(_E4M3_POS[-1])  # 448


def e4m3_decode(b) -> np.ndarray:
    """Value of each E4M3FN byte as float64 (NaN for 0x7F / 0xFF)."""
    return _E4M3_TABLE[np.asarray(b).astype(np.int64) & 0xFF]


def e4m3_encode(t) -> np.ndarray:
    """E4M3FN byte (uint8) nearest to each non-negative finite float32 ``t``.

    Definition: nearest non-negative finite E4M3 value, ties to the byte with
    mantissa LSB 0, values at or above 448 saturate to 0x7E.
    """
    t = np.asarray(t, dtype=np.float32)
    if not np.all(np.isfinite(t)) or np.any(t < 0):
        raise ValueError("e4m3_encode: expects finite non-negative input")
    a = t.astype(np.float64)
    vals = _E4M3_POS
    hi = np.minimum(np.searchsorted(vals, a, side="left"), len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = np.where(d_hi < d_lo, True, np.where(d_hi > d_lo, False, (hi & 1) == 0))
    pick_hi = np.where(hi == lo, True, pick_hi)
    return np.where(pick_hi, hi, lo).astype(np.uint8)
