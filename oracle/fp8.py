"""FP8 (E4M3, one scale per tensor), the baseline format of the pages,
written from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: gist.science, "Pretraining Large Language Models with NVFP4",
Resumen técnico §1 and §4 (NVFP4 is measured against an FP8 run of the same
model: validation loss and downstream accuracy); deultimominuto.info, "El
desafío de la cuantización" (FP8 as the current low-precision standard) and
"Cómo funciona NVFP4" (E4M3 named as the 8-bit format with 4 exponent and 3
mantissa bits).

The pages name FP8 only as the baseline and E4M3 as a format; they give no
scaling rule. Readings (the plainest per-tensor scaling, built from the same
steps the NVFP4 oracle takes for its tensor scale):

* F1 elements: one E4M3FN byte per element (bias 7, largest finite 448, no
  infinities), the same byte format as NVFP4's block scales; the sign bit is
  the sign of the scaled value, so -0.0 and negative values that round to 0
  give 0x80.
* F2 scale: one float32 decode scale per tensor, S8 = fp32(amax / 448), so
  the tensor's largest magnitude lands on E4M3's largest value. As for the
  NVFP4 tensor scale, S8 below 2^-100 (amax zero or vanishingly small) is
  replaced by 1.
* F3 element scaling: r = fp32(1 / S8) once per tensor, then y = fp32(x * r)
  per element (a reciprocal, then one multiply, the NVFP4 order), then the
  E4M3 byte nearest to |y|, ties to the even mantissa, saturating at 448.
* F4 layouts: the row copy is [R][C] bytes; the column copy (the transposed
  operand of the weight-gradient GEMM) is [C][R]. With one scale per tensor
  the bytes do not depend on the direction, so the column copy is the row
  copy transposed.
* F5 GEMM and dequantization: x_hat = fp32(e4m3(q) * S8);
  C = S8_a * S8_b * sum_k e4m3(qa[m][k]) * e4m3(qb[n][k]) (both operands
  K-contiguous, as the NVFP4 GEMM), computed here in float64 and rounded
  once to the output type.
"""

from __future__ import annotations

import numpy as np

from .formats import e4m3_decode, e4m3_encode

FP8_MAX = 448.0
_SCALE_FLOOR = np.float32(2.0 ** -100)


def fp8_tensor_scale(amax) -> np.float32:
    """F2: float32 decode scale of a tensor from its amax (float32, >= 0)."""
    a = np.float32(amax)
    if not np.isfinite(a) or a < 0:
        raise ValueError("fp8_tensor_scale: amax must be finite and >= 0")
    s = np.float32(a / np.float32(FP8_MAX))
    return np.float32(1.0) if s < _SCALE_FLOOR else s


def fp8_encode(y) -> np.ndarray:
    """F1/F3: E4M3FN bytes of float32 values y (sign bit from y's sign bit,
    magnitude nearest, ties to even, saturating at 448)."""
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("fp8_encode: non-finite input")
    sign = (y.view(np.uint32) >> 31).astype(np.uint8) << 7
    return (e4m3_encode(np.abs(y)) | sign).astype(np.uint8)


def fp8_quantize(x, amax=None):
    """F2-F4 for a float32 matrix x [R, C]. ``amax`` is the tensor amax when
    the caller supplies it (x may then be a slice of the tensor), else the
    largest magnitude of x.

    Returns (row codes [R][C] uint8, column codes [C][R] uint8, S8 float32)."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("fp8_quantize: non-finite input")
    if amax is None:
        amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    s8 = fp8_tensor_scale(amax)
    r = np.float32(np.float32(1.0) / s8)
    y = (x * r).astype(np.float32)  # float32 * float32 rounds once
    q = fp8_encode(y)
    return q, np.ascontiguousarray(q.T), s8


def fp8_dequantize(q, s8) -> np.ndarray:
    """F5: float32 values fp32(e4m3(q) * S8)."""
    v = e4m3_decode(np.asarray(q))
    return (v * np.float64(np.float32(s8))).astype(np.float32)


def fp8_gemm(qa, s8a, qb, s8b, out_dtype: str = "fp32") -> np.ndarray:
    """F5: C [M][N] = S8a * S8b * e4m3(qa) @ e4m3(qb)^T, float64, rounded once
    to float32 (out_dtype "fp32") or to bf16 through float32 ("bf16")."""
    a = e4m3_decode(np.asarray(qa))
    b = e4m3_decode(np.asarray(qb))
    if a.shape[1] != b.shape[1]:
        raise ValueError("fp8_gemm: K mismatch")
    c = (a @ b.T) * (np.float64(np.float32(s8a)) * np.float64(np.float32(s8b)))
    c32 = c.astype(np.float32)
    if out_dtype == "fp32":
        return c32
    if out_dtype == "bf16":
        import torch

        return torch.from_numpy(c32).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError("out_dtype must be fp32 or bf16")
