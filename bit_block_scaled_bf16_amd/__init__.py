"""NVFP4 quantizer and NVFP4 GEMM for AMD MI355X (gfx950).

Python side of the C-ABI library libnvfp4.so. ``_lib`` holds the entry points
with their C names (explicit output tensors); the helpers here allocate the
outputs with torch (device memory only) and call them. Every computation runs
in the library's HIP kernels; if the library is missing, importing the
binding's entry points raises.

The method: gist.science summary of "Pretraining Large Language Models with
NVFP4" (Resumen técnico §2) -- 16-element blocks with E4M3 scales and an FP32
tensor scale, 16x16 weight blocks, stochastic rounding of gradients, a 16x16
random Hadamard transform of the weight-gradient inputs, NVFP4 GEMMs.
"""

from __future__ import annotations

from dataclasses import dataclass

from . import _lib
from ._lib import (  # noqa: F401  (re-exported constants and raw entry points)
    AMAX_WS_BYTES,
    BF16,
    BLOCK_1D,
    BLOCK_2D,
    F32,
    OUT_COL,
    OUT_ROW,
    ROUND_RN,
    ROUND_SR,
    Nvfp4Error,
    nvfp4_dequantize,
    nvfp4_gemm,
    nvfp4_philox_fill,
    nvfp4_quantize,
    nvfp4_quantize_noalloc,
    nvfp4_quantize_row_rht,
    nvfp4_rht_quantize,
    nvfp4_rht_sign_mask,
    nvfp4_rht_transform,
    nvfp4_stream_copy,
    nvfp4_stream_read,
    mxfp4_dequantize,
    mxfp4_gemm,
    mxfp4_quantize,
    fp8_dequantize,
    fp8_gemm,
    fp8_quantize,
)

__all__ = [
    "NVFP4Tensor",
    "quantize",
    "rht_quantize",
    "quantize_row_rht",
    "dequantize",
    "gemm",
    "load",
]


def load():
    """Loads libnvfp4.so (raises ImportError when it has not been built)."""
    return _lib.lib()


@dataclass
class NVFP4Tensor:
    """One stored orientation of an NVFP4 matrix [rows][cols] (device)."""

    codes: "object"         # uint8 [rows, cols/2]
    scales: "object"        # uint8 [rows, cols/16] (1D) or [rows/16, cols/16] (2D)
    tensor_scale: "object"  # float32 [4]; element 0 is S
    block: int              # BLOCK_1D or BLOCK_2D
    rows: int
    cols: int


def _empty(shape, dtype, device):
    import torch

    return torch.empty(shape, dtype=dtype, device=device)


def _scalar(device):
    import torch

    return torch.zeros(4, dtype=torch.float32, device=device)


def amax_workspace(device):
    """A workspace for the tensor amax of one quantize call (its element 0
    holds the amax afterwards)."""
    import torch

    return torch.zeros(AMAX_WS_BYTES // 4, dtype=torch.float32, device=device)


def quantize(x, block: int = BLOCK_1D, rounding: int = ROUND_RN, seed: int = 0, offset: int = 0,
             outputs: int = OUT_ROW | OUT_COL, amax=None, dev_status=None):
    """Quantizes x [rows, cols] (bf16 or float32, device).

    Returns (row copy or None, column copy or None, amax workspace or None).
    The column copy is stored as the quantized transpose [cols, rows/2].
    """
    import torch

    rows, cols = x.shape
    dev = x.device
    scale = _scalar(dev)
    ws = None if amax is not None else amax_workspace(dev)
    row = col = None
    q_row = s_row = q_col = s_col = None
    two_d = block == BLOCK_2D
    if outputs & OUT_ROW:
        q_row = _empty((rows, cols // 2), torch.uint8, dev)
        s_row = _empty((rows // 16, cols // 16) if two_d else (rows, cols // 16), torch.uint8, dev)
        row = NVFP4Tensor(q_row, s_row, scale, block, rows, cols)
    if outputs & OUT_COL:
        q_col = _empty((cols, rows // 2), torch.uint8, dev)
        s_col = _empty((cols // 16, rows // 16) if two_d else (cols, rows // 16), torch.uint8, dev)
        col = NVFP4Tensor(q_col, s_col, scale, block, cols, rows)
    nvfp4_quantize(x, block, rounding, seed, offset, outputs, amax, ws, q_row, s_row, q_col,
                   s_col, scale, dev_status)
    return row, col, ws


def rht_quantize(x, rht_seed: int, rounding: int = ROUND_RN, seed: int = 0, offset: int = 0,
                 amax=None, dev_status=None):
    """Hadamard transform along tokens + 16x1 quantization of x [tokens, cols].

    Returns (NVFP4Tensor [cols, tokens], amax workspace or None).
    """
    import torch

    tokens, cols = x.shape
    dev = x.device
    scale = _scalar(dev)
    ws = None if amax is not None else amax_workspace(dev)
    q = _empty((cols, tokens // 2), torch.uint8, dev)
    s = _empty((cols, tokens // 16), torch.uint8, dev)
    nvfp4_rht_quantize(x, rht_seed, rounding, seed, offset, amax, ws, q, s, scale, dev_status)
    return NVFP4Tensor(q, s, scale, BLOCK_1D, cols, tokens), ws


def quantize_row_rht(x, rht_seed: int, rounding_t: int = ROUND_RN, seed: int = 0,
                     offset: int = 0, amax=None, dev_status=None):
    """Both copies of an activation x [tokens, cols] from one read: the 1x16
    row copy (round to nearest) and the Hadamard 16x1 column copy, each with
    its own tensor scale. ``amax`` is None or 2 floats (amax of x, amax of the
    transformed x).

    Returns (row NVFP4Tensor [tokens, cols], column NVFP4Tensor [cols, tokens],
    amax workspace or None).
    """
    import torch

    tokens, cols = x.shape
    dev = x.device
    scale_row, scale_t = _scalar(dev), _scalar(dev)
    ws = None if amax is not None else amax_workspace(dev)
    q_row = _empty((tokens, cols // 2), torch.uint8, dev)
    s_row = _empty((tokens, cols // 16), torch.uint8, dev)
    q_t = _empty((cols, tokens // 2), torch.uint8, dev)
    s_t = _empty((cols, tokens // 16), torch.uint8, dev)
    nvfp4_quantize_row_rht(x, rht_seed, rounding_t, seed, offset, amax, ws, q_row, s_row,
                           scale_row, q_t, s_t, scale_t, dev_status)
    return (NVFP4Tensor(q_row, s_row, scale_row, BLOCK_1D, tokens, cols),
            NVFP4Tensor(q_t, s_t, scale_t, BLOCK_1D, cols, tokens), ws)


def dequantize(t: NVFP4Tensor, out_dtype=None):
    """Float32 (default) or bf16 values of an NVFP4 tensor."""
    import torch

    out_dtype = torch.float32 if out_dtype is None else out_dtype
    y = _empty((t.rows, t.cols), out_dtype, t.codes.device)
    nvfp4_dequantize(t.codes, t.scales, t.tensor_scale, t.rows, t.cols, t.block, y)
    return y


def gemm(a: NVFP4Tensor, b: NVFP4Tensor, out_dtype=None, out=None):
    """C = deq(a) @ deq(b)^T, float32 accumulation, bf16 output by default."""
    import torch

    if a.cols != b.cols:
        raise ValueError("a and b must share K")
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    c = out if out is not None else _empty((a.rows, b.rows), out_dtype, a.codes.device)
    nvfp4_gemm(a.codes, a.scales, a.tensor_scale, a.block, b.codes, b.scales, b.tensor_scale,
               b.block, a.rows, b.rows, a.cols, c)
    return c


# ---------------------------------------------------------------------------
# MXFP4, the comparison format: 32-element blocks along rows, E8M0 scales.
# ---------------------------------------------------------------------------


def mx_quantize(x):
    """MXFP4 codes [rows, cols/2] and E8M0 scale bytes [rows, cols/32] of x."""
    import torch

    rows, cols = x.shape
    q = _empty((rows, cols // 2), torch.uint8, x.device)
    s = _empty((rows, cols // 32), torch.uint8, x.device)
    mxfp4_quantize(x, q, s)
    return q, s


def mx_dequantize(q, s, out_dtype=None):
    import torch

    out_dtype = torch.float32 if out_dtype is None else out_dtype
    rows, cols = q.shape[0], q.shape[1] * 2
    y = _empty((rows, cols), out_dtype, q.device)
    mxfp4_dequantize(q, s, rows, cols, y)
    return y


def mx_gemm(qa, sa, qb, sb, out_dtype=None, out=None):
    """C = deq(A) @ deq(B)^T for MXFP4 operands [M, K] and [N, K]."""
    import torch

    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    m, n, k = qa.shape[0], qb.shape[0], qa.shape[1] * 2
    c = out if out is not None else _empty((m, n), out_dtype, qa.device)
    mxfp4_gemm(qa, sa, qb, sb, m, n, k, c)
    return c


# ---------------------------------------------------------------------------
# FP8 (E4M3, one scale per tensor), the baseline format.
# ---------------------------------------------------------------------------


def f8_quantize(x, outputs: int = OUT_ROW, amax_ws=None):
    """FP8 copies of x: (row bytes [rows, cols] or None, column bytes
    [cols, rows] or None, decode scale S8 as a float32 [4] tensor)."""
    import torch

    rows, cols = x.shape
    q_row = _empty((rows, cols), torch.uint8, x.device) if outputs & OUT_ROW else None
    q_col = _empty((cols, rows), torch.uint8, x.device) if outputs & OUT_COL else None
    ts = _scalar(x.device)
    ws = amax_ws if amax_ws is not None else amax_workspace(x.device)
    fp8_quantize(x, outputs, None, ws, q_row, q_col, ts)
    return q_row, q_col, ts


def f8_dequantize(q, tensor_scale, out_dtype=None):
    import torch

    out_dtype = torch.float32 if out_dtype is None else out_dtype
    rows, cols = q.shape
    y = _empty((rows, cols), out_dtype, q.device)
    fp8_dequantize(q, tensor_scale, rows, cols, y)
    return y


def f8_gemm(qa, ta, qb, tb, out_dtype=None, out=None):
    """C = S8_a S8_b e4m3(A) @ e4m3(B)^T for FP8 operands [M, K] and [N, K]."""
    import torch

    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    m, n, k = qa.shape[0], qb.shape[0], qa.shape[1]
    c = out if out is not None else _empty((m, n), out_dtype, qa.device)
    fp8_gemm(qa, ta, qb, tb, m, n, k, c)
    return c
