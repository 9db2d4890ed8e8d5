"""ctypes binding of libnvfp4.so (the C ABI declared in include/nvfp4.h).

The functions named like the C entry points take torch tensors (device
memory) or None and only marshal arguments: every computation runs in the
HIP kernels of the library. Work is enqueued on torch's current HIP stream.
A missing library raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libnvfp4.so")

# Status codes / enums (include/nvfp4.h)
OK, ERR_NULL, ERR_SHAPE, ERR_ENUM, ERR_ALIGN, ERR_HIP = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1
BLOCK_1D, BLOCK_2D = 0, 1
ROUND_RN, ROUND_SR = 0, 1
OUT_ROW, OUT_COL = 1, 2

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32
_INT = ctypes.c_int

_SIGNATURES = {
    "nvfp4_quantize": (_INT, [_P, _INT, _I64, _I64, _I64, _INT, _INT, _U64, _U32, _INT, _P, _P,
                              _P, _P, _P, _P, _P, _P, _P]),
    "nvfp4_quantize_noalloc": (_INT, [_P, _INT, _I64, _I64, _I64, _INT, _INT, _U64, _U32, _INT,
                                      _P, _P, _P, _P, _P, _P, _P, _P]),
    "nvfp4_rht_quantize": (_INT, [_P, _INT, _I64, _I64, _I64, _U64, _INT, _U64, _U32, _P, _P, _P,
                                  _P, _P, _P, _P]),
    "nvfp4_quantize_row_rht": (_INT, [_P, _INT, _I64, _I64, _I64, _U64, _INT, _U64, _U32, _P,
                                      _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "nvfp4_dequantize": (_INT, [_P, _P, _P, _I64, _I64, _INT, _INT, _P, _I64, _P]),
    "nvfp4_gemm": (_INT, [_P, _P, _P, _INT, _P, _P, _P, _INT, _I64, _I64, _I64, _P, _INT, _I64,
                          _P]),
    "nvfp4_philox_fill": (_INT, [_U64, _U32, _U32, _I64, _P, _P]),
    "nvfp4_rht_transform": (_INT, [_P, _INT, _I64, _I64, _I64, _U64, _P, _P]),
    "nvfp4_rht_sign_mask": (_U32, [_U64]),
    "nvfp4_status_string": (ctypes.c_char_p, [_INT]),
    "mxfp4_quantize": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P]),
    "mxfp4_dequantize": (_INT, [_P, _P, _I64, _I64, _INT, _P, _I64, _P]),
    "mxfp4_gemm": (_INT, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _INT, _I64, _P]),
    "fp8_quantize": (_INT, [_P, _INT, _I64, _I64, _I64, _INT, _P, _P, _P, _P, _P, _P, _P]),
    "fp8_dequantize": (_INT, [_P, _P, _I64, _I64, _INT, _P, _I64, _P]),
    "fp8_gemm": (_INT, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _INT, _I64, _P]),
    "nvfp4_stream_read": (_INT, [_P, _I64, _P, _P]),
    "nvfp4_stream_copy": (_INT, [_P, _P, _I64, _P]),
}

EXPORTED = tuple(_SIGNATURES)

# Bytes of the amax workspace (NVFP4_AMAX_WS_BYTES in include/nvfp4.h).
AMAX_WS_BYTES = 16384
# Words of nvfp4_stream_read's checksum buffer (NVFP4_STREAM_SINK_WORDS).
STREAM_SINK_WORDS = 1024

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().nvfp4_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m bit_block_scaled_bf16_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _ws(t) -> int | None:
    """Pointer of an amax workspace, which must hold AMAX_WS_BYTES (the
    library would write past a smaller one)."""
    if t is None:
        return None
    if t.numel() * t.element_size() < AMAX_WS_BYTES or not t.is_contiguous():
        raise ValueError(f"amax workspace must be a contiguous buffer of >= {AMAX_WS_BYTES} bytes")
    return t.data_ptr()


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch

    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise Nvfp4Error(fn, status)


def _ld(t) -> int:
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with unit column stride")
    if t.shape[0] <= 1:
        return max(t.stride(0), t.shape[1])  # the stride of a size-1 dim is arbitrary
    return t.stride(0)


# ---------------------------------------------------------------------------
# Entry points with the C names (explicit output tensors).
# ---------------------------------------------------------------------------


def nvfp4_quantize(x, block, rounding, seed, offset, outputs, amax_in, amax_ws, q_row, s_row,
                   q_col, s_col, tensor_scale, dev_status=None, stream=None) -> None:
    rows, cols = x.shape
    _check("nvfp4_quantize", lib().nvfp4_quantize(
        _ptr(x), _dtype_code(x), rows, cols, _ld(x), block, rounding, seed, offset, outputs,
        _ptr(amax_in), _ws(amax_ws), _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col),
        _ptr(tensor_scale), _ptr(dev_status), _stream(stream)))


def nvfp4_quantize_noalloc(x, block, rounding, seed, offset, outputs, amax_in, q_row, s_row,
                           q_col, s_col, tensor_scale, dev_status=None, stream=None) -> None:
    rows, cols = x.shape
    _check("nvfp4_quantize_noalloc", lib().nvfp4_quantize_noalloc(
        _ptr(x), _dtype_code(x), rows, cols, _ld(x), block, rounding, seed, offset, outputs,
        _ptr(amax_in), _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col), _ptr(tensor_scale),
        _ptr(dev_status), _stream(stream)))


def nvfp4_rht_quantize(x, rht_seed, rounding, seed, offset, amax_in, amax_ws, q_t, s_t,
                       tensor_scale, dev_status=None, stream=None) -> None:
    tokens, cols = x.shape
    _check("nvfp4_rht_quantize", lib().nvfp4_rht_quantize(
        _ptr(x), _dtype_code(x), tokens, cols, _ld(x), rht_seed, rounding, seed, offset,
        _ptr(amax_in), _ws(amax_ws), _ptr(q_t), _ptr(s_t), _ptr(tensor_scale),
        _ptr(dev_status), _stream(stream)))


def nvfp4_quantize_row_rht(x, rht_seed, rounding_t, seed, offset, amax_in, amax_ws, q_row, s_row,
                           tensor_scale_row, q_t, s_t, tensor_scale_t, dev_status=None,
                           stream=None) -> None:
    tokens, cols = x.shape
    _check("nvfp4_quantize_row_rht", lib().nvfp4_quantize_row_rht(
        _ptr(x), _dtype_code(x), tokens, cols, _ld(x), rht_seed, rounding_t, seed, offset,
        _ptr(amax_in), _ws(amax_ws), _ptr(q_row), _ptr(s_row), _ptr(tensor_scale_row),
        _ptr(q_t), _ptr(s_t), _ptr(tensor_scale_t), _ptr(dev_status), _stream(stream)))


def nvfp4_dequantize(q, s, tensor_scale, rows, cols, block, y, stream=None) -> None:
    _check("nvfp4_dequantize", lib().nvfp4_dequantize(
        _ptr(q), _ptr(s), _ptr(tensor_scale), rows, cols, block, _dtype_code(y), _ptr(y), _ld(y),
        _stream(stream)))


def nvfp4_gemm(qa, sa, ta, a_block, qb, sb, tb, b_block, M, N, K, c, stream=None) -> None:
    _check("nvfp4_gemm", lib().nvfp4_gemm(
        _ptr(qa), _ptr(sa), _ptr(ta), a_block, _ptr(qb), _ptr(sb), _ptr(tb), b_block, M, N, K,
        _ptr(c), _dtype_code(c), _ld(c), _stream(stream)))


def mxfp4_quantize(x, q, s, stream=None) -> None:
    rows, cols = x.shape
    _check("mxfp4_quantize", lib().mxfp4_quantize(
        _ptr(x), _dtype_code(x), rows, cols, _ld(x), _ptr(q), _ptr(s), _stream(stream)))


def mxfp4_dequantize(q, s, rows, cols, y, stream=None) -> None:
    _check("mxfp4_dequantize", lib().mxfp4_dequantize(
        _ptr(q), _ptr(s), rows, cols, _dtype_code(y), _ptr(y), _ld(y), _stream(stream)))


def mxfp4_gemm(qa, sa, qb, sb, M, N, K, c, stream=None) -> None:
    _check("mxfp4_gemm", lib().mxfp4_gemm(
        _ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), M, N, K, _ptr(c), _dtype_code(c), _ld(c),
        _stream(stream)))


def fp8_quantize(x, outputs, amax_in, amax_ws, q_row, q_col, tensor_scale, dev_status=None,
                 stream=None) -> None:
    rows, cols = x.shape
    _check("fp8_quantize", lib().fp8_quantize(
        _ptr(x), _dtype_code(x), rows, cols, _ld(x), outputs, _ptr(amax_in), _ws(amax_ws),
        _ptr(q_row), _ptr(q_col), _ptr(tensor_scale), _ptr(dev_status), _stream(stream)))


def fp8_dequantize(q, tensor_scale, rows, cols, y, stream=None) -> None:
    _check("fp8_dequantize", lib().fp8_dequantize(
        _ptr(q), _ptr(tensor_scale), rows, cols, _dtype_code(y), _ptr(y), _ld(y), _stream(stream)))


def fp8_gemm(qa, ta, qb, tb, M, N, K, c, stream=None) -> None:
    _check("fp8_gemm", lib().fp8_gemm(
        _ptr(qa), _ptr(ta), _ptr(qb), _ptr(tb), M, N, K, _ptr(c), _dtype_code(c), _ld(c),
        _stream(stream)))


def nvfp4_philox_fill(seed, c2, c3, n_groups, out, stream=None) -> None:
    _check("nvfp4_philox_fill", lib().nvfp4_philox_fill(seed, c2, c3, n_groups, _ptr(out),
                                                        _stream(stream)))


def nvfp4_rht_transform(x, rht_seed, out, stream=None) -> None:
    tokens, cols = x.shape
    _check("nvfp4_rht_transform", lib().nvfp4_rht_transform(
        _ptr(x), _dtype_code(x), tokens, cols, _ld(x), rht_seed, _ptr(out), _stream(stream)))


def nvfp4_rht_sign_mask(rht_seed: int) -> int:
    return int(lib().nvfp4_rht_sign_mask(rht_seed))


def nvfp4_stream_read(src, nbytes, sink, stream=None) -> None:
    if sink.numel() * sink.element_size() < 4 * STREAM_SINK_WORDS:
        raise ValueError(f"stream_read sink must hold {STREAM_SINK_WORDS} uint32")
    _check("nvfp4_stream_read", lib().nvfp4_stream_read(_ptr(src), nbytes, _ptr(sink),
                                                        _stream(stream)))


def nvfp4_stream_copy(src, dst, nbytes, stream=None) -> None:
    _check("nvfp4_stream_copy", lib().nvfp4_stream_copy(_ptr(src), _ptr(dst), nbytes,
                                                        _stream(stream)))
