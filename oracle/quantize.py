"""NVFP4 quantization with two-level scaling, its dequantization and layouts.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* gist.science, "Pretraining Large Language Models with NVFP4", Resumen
  técnico §2 "Formato NVFP4": blocks of 16 elements (MXFP4 uses 32), a
  per-tensor FP32 scale plus a per-block E4M3 scale, so the block maximum is
  represented more precisely than with power-of-two scales.
* Same page, §2 "Escalado Bidimensional (2D) y Redondeo Estocástico": weights
  use 16x16 blocks so that the forward and backward passes use the same
  quantized weights; stochastic rounding only for gradients.
* Same page, Lo esencial, item 1: small blocks keep a large value from
  wiping out the small ones of other blocks; a tensor-wide scale keeps
  everything in range.

Readings, in the order the computation runs (numbers refer to float32
operations, each rounded to nearest even):

1. Tensor amax ``A = max |x|`` (exact).
2. Tensor scale ``S = A / 2688`` (2688 = 6 * 448: the largest E2M1 magnitude
   times the largest E4M3 value, so the largest block scale and the largest
   element both use the top of their ranges). If S < 2^-100 (A is zero or
   vanishingly small) S is set to 1, which makes every block scale 0 and the
   whole tensor zero. A non-finite A is an error.
3. Block amax ``a_b = max |x|`` over the 16 (or 16x16) block elements.
4. Block scale byte ``s_b = E4M3(a_b / (6 * S))`` (two float32 operations,
   then round to nearest even with saturation at 448).
5. ``s_f = value(s_b)``; if s_f == 0 every code of the block is 0x0;
   otherwise the block multiplier is ``r = 1 / (s_f * S)`` (two operations).
6. ``y = x * r`` (one operation per element).
7. ``q = E2M1_RN(y)`` or ``E2M1_SR(y, u16)`` (see ``formats``).
8. Packing: byte j of a row holds element 2j in its low nibble and element
   2j+1 in its high nibble. Scales are one byte each, row-major.

Layouts:
* row-blocked copy of an R x C matrix (blocks of 1x16 along C): codes
  [R][C/2], scales [R][C/16];
* column-blocked copy (blocks of 16x1 along R), stored as the quantized
  transpose: codes [C][R/2], scales [C][R/16];
* 16x16 blocks: codes [R][C/2] and the transposed codes [C][R/2], scale grid
  [R/16][C/16] and its transpose [C/16][R/16].
Dequantized value: ``x_hat = (e2m1(q) * s_f) * S`` (two float32 operations;
the first is exact).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import e2m1_decode, e2m1_encode_rn, e2m1_encode_sr, e4m3_decode, e4m3_encode
from .hadamard import rht
from .philox import STREAM_COL, STREAM_ROW, sr_random_u16

E2M1_MAX = np.float32(6.0)
E4M3_MAX = np.float32(448.0)
TENSOR_SCALE_DIVISOR = np.float32(6.0 * 448.0)  # 2688
TENSOR_SCALE_FLOOR = np.float32(2.0**-100)


@dataclass
class QuantizedTensor:
    """One stored orientation of an NVFP4 tensor."""

    codes: np.ndarray  # uint8 [rows][cols/2], two codes per byte
    scales: np.ndarray  # uint8, [rows][cols/16] (1x16) or [rows/16][cols/16] (16x16)
    tensor_scale: np.float32  # S, the decode scale
    amax: np.float32  # tensor amax the scale came from
    block: str  # "1d" or "2d"


def tensor_scale(amax) -> np.float32:
    """Step 2: float32 tensor decode scale from the tensor amax."""
    a = np.float32(amax)
    if not np.isfinite(a):
        raise ValueError("tensor amax is not finite")
    s = np.float32(a / TENSOR_SCALE_DIVISOR)
    if s < TENSOR_SCALE_FLOOR:
        s = np.float32(1.0)
    return s


def _block_multiplier(amax_b: np.ndarray, s: np.float32):
    """Steps 4-5 for an array of block amaxes: scale bytes, their values and
    the encode multipliers (0 where the block scale is 0)."""
    amax_b = np.asarray(amax_b, dtype=np.float32)
    denom = np.float32(np.float32(6.0) * s)
    t = (amax_b / denom).astype(np.float32)
    s_b = e4m3_encode(t)
    s_f = e4m3_decode(s_b).astype(np.float32)  # exact in float32
    nz = s_f != 0
    prod = (s_f * s).astype(np.float32)
    r = np.where(nz, np.float32(1.0) / np.where(nz, prod, np.float32(1.0)), np.float32(0.0))
    return s_b, s_f, r.astype(np.float32), nz


def _round_codes(y: np.ndarray, rounding: str, u16) -> np.ndarray:
    if rounding == "rn":
        return e2m1_encode_rn(y)
    if rounding == "sr":
        return e2m1_encode_sr(y, u16)
    raise ValueError(f"unknown rounding {rounding!r}")


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[R, C] codes (0..15) -> [R, C/2] bytes, even element in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[R, C/2] bytes -> [R, C] codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def quantize_rows(m, s: np.float32, rounding: str = "rn", seed: int = 0, offset: int = 0,
                  stream: int = STREAM_ROW, index_base: int = 0):
    """Steps 3-7 for a float32 matrix m [R, C] with 1x16 blocks along C.

    Returns (codes [R, C] unpacked uint8, scale bytes [R, C/16]).
    For SR the element index is ``index_base`` plus the row-major index of m
    (index_base lets a caller quantize a few rows of a larger stored matrix).
    """
    m = np.asarray(m, dtype=np.float32)
    r_, c_ = m.shape
    if c_ % 16 != 0:
        raise ValueError("columns must be a multiple of 16")
    blocks = m.reshape(r_, c_ // 16, 16)
    amax_b = np.max(np.abs(blocks), axis=2)
    s_b, _, r, nz = _block_multiplier(amax_b, s)
    y = (blocks * r[:, :, None]).astype(np.float32)
    u16 = None
    if rounding == "sr":
        e = (np.int64(index_base) + np.arange(r_ * c_, dtype=np.int64)).reshape(r_, c_ // 16, 16)
        u16 = sr_random_u16(seed, offset, stream, e)
    codes = _round_codes(y, rounding, u16)
    codes = np.where(nz[:, :, None], codes, np.uint8(0)).astype(np.uint8)
    return codes.reshape(r_, c_), s_b


def _as_float32(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise ValueError("oracle inputs are float32 arrays (bf16 data widened exactly)")
    return x


def quantize(x, rounding: str = "rn", seed: int = 0, offset: int = 0,
             outputs=("row", "col"), amax=None) -> dict:
    """1x16 / 16x1 quantization of a float32 [R, C] matrix.

    outputs: any of "row" (blocks along C) and "col" (blocks along R, stored
    transposed). Both copies share the tensor scale. ``amax`` overrides the
    computed tensor amax (a caller-supplied amax).
    Returns {"row": QuantizedTensor, "col": QuantizedTensor} (requested ones).
    """
    x = _as_float32(x)
    a = np.float32(np.max(np.abs(x))) if amax is None else np.float32(amax)
    s = tensor_scale(a)
    out = {}
    if "row" in outputs:
        codes, sb = quantize_rows(x, s, rounding, seed, offset, STREAM_ROW)
        out["row"] = QuantizedTensor(pack_codes(codes), sb, s, a, "1d")
    if "col" in outputs:
        codes, sb = quantize_rows(np.ascontiguousarray(x.T), s, rounding, seed, offset, STREAM_COL)
        out["col"] = QuantizedTensor(pack_codes(codes), sb, s, a, "1d")
    return out


def quantize_2d(x, amax=None) -> dict:
    """16x16-block quantization (weights, round to nearest) of float32 [R, C].

    Returns {"row": codes [R][C/2] + grid [R/16][C/16],
             "col": codes [C][R/2] + grid^T [C/16][R/16]}.
    """
    x = _as_float32(x)
    r_, c_ = x.shape
    if r_ % 16 or c_ % 16:
        raise ValueError("2D blocks need both dimensions to be multiples of 16")
    a = np.float32(np.max(np.abs(x))) if amax is None else np.float32(amax)
    s = tensor_scale(a)
    tiles = x.reshape(r_ // 16, 16, c_ // 16, 16)
    amax_b = np.max(np.abs(tiles), axis=(1, 3))  # [R/16, C/16]
    s_b, _, r, nz = _block_multiplier(amax_b, s)
    y = (tiles * r[:, None, :, None]).astype(np.float32)
    codes = e2m1_encode_rn(y)
    codes = np.where(nz[:, None, :, None], codes, np.uint8(0)).astype(np.uint8).reshape(r_, c_)
    return {
        "row": QuantizedTensor(pack_codes(codes), s_b, s, a, "2d"),
        "col": QuantizedTensor(pack_codes(np.ascontiguousarray(codes.T)),
                               np.ascontiguousarray(s_b.T), s, a, "2d"),
    }


def rht_quantize(x, rht_seed: int, rounding: str = "rn", seed: int = 0, offset: int = 0,
                 amax=None) -> QuantizedTensor:
    """Weight-gradient operand path: RHT along tokens, then 16x1 blocks along
    tokens, stored transposed. x: float32 [T, C]. The tensor amax is the amax
    of the transformed tensor. Returns codes [C][T/2], scales [C][T/16]."""
    x = _as_float32(x)
    xt = rht(x, rht_seed)  # float32 [T, C]
    a = np.float32(np.max(np.abs(xt))) if amax is None else np.float32(amax)
    s = tensor_scale(a)
    codes, sb = quantize_rows(np.ascontiguousarray(xt.T), s, rounding, seed, offset, STREAM_COL)
    return QuantizedTensor(pack_codes(codes), sb, s, a, "1d")


def dequantize(codes_packed, scales, s, block: str = "1d") -> np.ndarray:
    """float32 [R, C] values of a stored orientation: (e2m1(q) * s_f) * S."""
    codes = unpack_codes(codes_packed)
    r_, c_ = codes.shape
    scales = np.asarray(scales, dtype=np.uint8)
    s_f = e4m3_decode(scales).astype(np.float32)
    if block == "1d":
        if scales.shape != (r_, c_ // 16):
            raise ValueError("1d scales must be [R, C/16]")
        sf_full = np.repeat(s_f, 16, axis=1)
    elif block == "2d":
        if scales.shape != (r_ // 16, c_ // 16):
            raise ValueError("2d scales must be [R/16, C/16]")
        sf_full = np.repeat(np.repeat(s_f, 16, axis=0), 16, axis=1)
    else:
        raise ValueError(f"unknown block {block!r}")
    v = e2m1_decode(codes).astype(np.float32)
    return ((v * sf_full).astype(np.float32) * np.float32(s)).astype(np.float32)
