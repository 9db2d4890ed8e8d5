"""Reference for the GEMM that consumes NVFP4 operands.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: gist.science, "Pretraining Large Language Models with NVFP4",
Resumen técnico §2 "Precisión Mixta Selectiva" -- apart from a small share of
layers kept in BF16, the GEMMs of the linear layers run on NVFP4 operands;
§2 "Formato NVFP4" -- the format has native Tensor Core support on the
hardware the report used.

Reading: the GEMM is C = deq(A) @ deq(B)^T with A [M, K] and B [N, K] both
blocked along K, where deq is the float32 dequantization
``(e2m1(q) * s_f) * S``. The oracle dequantizes each operand in float32
(``quantize.dequantize``) and multiplies in float64 (a library matmul), with
no blocking or reordering of its own. The result is float64; callers round it
to the output type they compare against.
"""

from __future__ import annotations

import numpy as np

from .quantize import dequantize


def gemm(a_codes, a_scales, a_s, a_block: str,
         b_codes, b_scales, b_s, b_block: str) -> np.ndarray:
    """C[M, N] (float64) = deq(A) @ deq(B)^T."""
    a = dequantize(a_codes, a_scales, a_s, a_block).astype(np.float64)
    b = dequantize(b_codes, b_scales, b_s, b_block).astype(np.float64)
    if a.shape[1] != b.shape[1]:
        raise ValueError("A and B must share K")
    return a @ b.T
