"""MXFP4, the comparison format of the pages, written from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: gist.science, "Pretraining Large Language Models with NVFP4",
Resumen técnico §2 "Formato NVFP4" (MXFP4 quantizes in blocks of 32
elements, NVFP4 in blocks of 16) and §1 (MXFP4's limited scale factors cost
dynamic range and precision); deultimominuto.info, "Cómo funciona NVFP4"
(the same comparison).

The pages give only the block size and that the scales are coarser than
NVFP4's E4M3. Readings (the usual microscaling definition of the format):

* M1 block: 32 consecutive elements along a row (the GEMM K dimension), one
  scale byte each; elements are the same E2M1 codes as NVFP4's.
* M2 scale: E8M0, an unsigned 8-bit exponent with value 2^(b - 127) for
  b = 0..254 (255 would be NaN and is never produced). No tensor scale.
* M3 scale choice: b = max(floor(log2(amax_b)) - 2 + 127, 0), so the block
  amax maps into [4, 8) (2 is the exponent of E2M1's largest binade);
  amax_b = 0 gives b = 0.
* M4 elements: y = x / 2^(b - 127) (a power-of-two scaling), then the NVFP4
  round-to-nearest rule (ties to the even code, saturation at 6). A block
  amax in (6, 8) * 2^(b - 127) therefore clips to 6: the price of power-of-
  two scales.
* M5 round to nearest only (the comparison is of the format, not of SR).
"""

from __future__ import annotations

import numpy as np

from .formats import e2m1_decode, e2m1_encode_rn
from .quantize import pack_codes, unpack_codes

MX_BLOCK = 32


def e8m0_decode(b) -> np.ndarray:
    """Value of E8M0 scale bytes (float64; NaN for 255)."""
    b = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def mx_scale_bytes(amax) -> np.ndarray:
    """M3: E8M0 byte of each block amax (float32 array, >= 0, finite)."""
    a = np.asarray(amax, dtype=np.float64)
    if np.any(~np.isfinite(a)) or np.any(a < 0):
        raise ValueError("mx_scale_bytes: amax must be finite and >= 0")
    _, e = np.frexp(a)  # a = m * 2^e, m in [0.5, 1): floor(log2 a) = e - 1 (exact)
    b = (e - 1) - 2 + 127
    b = np.where(a > 0, b, 0)
    return np.clip(b, 0, 254).astype(np.uint8)


def mx_quantize(x) -> tuple[np.ndarray, np.ndarray]:
    """M1-M5 for a float32 matrix x [R, C], C % 32 == 0.

    Returns (codes [R][C/2], two per byte with the even element in the low
    nibble, as NVFP4; scales [R][C/32] E8M0 bytes)."""
    x = np.asarray(x, dtype=np.float32)
    r_, c_ = x.shape
    if c_ % MX_BLOCK:
        raise ValueError("columns must be a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("mx_quantize: non-finite input")
    blocks = x.reshape(r_, c_ // MX_BLOCK, MX_BLOCK).astype(np.float64)
    amax = np.max(np.abs(blocks), axis=2)
    b = mx_scale_bytes(amax)
    y = blocks * np.ldexp(1.0, 127 - b.astype(np.int64))[:, :, None]  # exact
    codes = e2m1_encode_rn(y.astype(np.float32).reshape(r_, c_))
    return pack_codes(codes), b


def mx_dequantize(codes_packed, scales) -> np.ndarray:
    """float32 [R, C] values: e2m1(q) * 2^(b - 127)."""
    q = unpack_codes(codes_packed)
    r_, c_ = q.shape
    v = e2m1_decode(q).reshape(r_, c_ // MX_BLOCK, MX_BLOCK)
    v = v * e8m0_decode(np.asarray(scales))[:, :, None]
    return v.reshape(r_, c_).astype(np.float32)


def mx_gemm(qa, sa, qb, sb) -> np.ndarray:
    """C[M][N] = sum_k deq(A)[m][k] deq(B)[n][k] in float64 (both operands
    K-contiguous, as stored)."""
    a = mx_dequantize(qa, sa).astype(np.float64)
    b = mx_dequantize(qb, sb).astype(np.float64)
    return a @ b.T
