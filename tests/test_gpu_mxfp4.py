"""GPU parity of the MXFP4 comparison path with the oracle: the 1x32
quantizer's codes and E8M0 scale bytes and the dequantizer bit for bit; the
GEMM on the block-scaled FP4 MFMA within the bound of the NVFP4 GEMM tests
(relative Frobenius error <= 1e-2 plus the per-element bound of float32
accumulation of exact products and a final rounding)."""

import numpy as np
import pytest

import oracle as o
import workloads as wl
from tests._helpers import announce, host, require_gpu, to_device
from tests.test_gpu_gemm import check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows,cols", [(1, 32), (8, 64), (37, 1024), (300, 5120)])
def test_mx_quantize_parity(dtype, rows, cols):
    require_gpu()
    import bit_block_scaled_bf16_amd as nv

    announce(f"mx quantize {rows}x{cols} {dtype}")
    x = wl.normal((rows, cols), seed=rows + cols, outlier_channels=min(4, cols // 32),
                  dtype=dtype)
    q, s = nv.mx_quantize(to_device(x, dtype))
    rq, rs = o.mx_quantize(x)
    assert np.array_equal(host(s), rs)
    assert np.array_equal(host(q), rq)
    import torch

    for out in (torch.float32, torch.bfloat16):
        d = host(nv.mx_dequantize(q, s, out).float())
        assert np.array_equal(d, o.mx_dequantize(rq, rs))


def test_mx_quantize_padded_rows_and_extremes():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x = wl.normal((64, 96), seed=9, dtype="fp32")
    x[0, :32] = 0.0                        # zero block: scale byte 0, codes 0
    x[1, :32] *= np.float32(2.0 ** -120)   # tiny block
    x[2, :32] *= np.float32(2.0 ** 100)    # huge block
    x[3, 5] = np.float32(7.5)              # amax that clips to 6 after scaling
    big = np.zeros((64, 160), np.float32)
    big[:, :96] = x
    xd = to_device(big, "fp32")[:, :96]
    q, s = nv.mx_quantize(xd)
    rq, rs = o.mx_quantize(x)
    assert np.array_equal(host(s), rs) and np.array_equal(host(q), rq)


@pytest.mark.parametrize("m,n,k", [(32, 32, 128), (256, 256, 128), (300, 520, 256),
                                   (512, 768, 1024), (33, 47, 384), (2500, 2608, 512),
                                   (272, 256, 5120), (3072, 6144, 256)])
def test_mx_gemm_parity(m, n, k):
    """(3072, 6144, 256): 12 x 24 tiles, nine 4 x 8 tile blocks: eight handed
    to the XCDs together, one after them in plain order."""
    require_gpu()
    import torch

    import bit_block_scaled_bf16_amd as nv

    announce(f"mx gemm {m}x{n}x{k}")
    a = wl.normal((m, k), seed=m + k, outlier_channels=4 if k >= 256 else 0)
    b = wl.normal((n, k), seed=n + k + 1)
    qa, sa = nv.mx_quantize(to_device(a, "bf16"))
    qb, sb = nv.mx_quantize(to_device(b, "bf16"))
    ra = o.mx_dequantize(host(qa), host(sa)).astype(np.float64)
    rb = o.mx_dequantize(host(qb), host(sb)).astype(np.float64)
    ref, absref = ra @ rb.T, np.abs(ra) @ np.abs(rb).T
    check(host(nv.mx_gemm(qa, sa, qb, sb).float()), ref, absref, k)
    check(host(nv.mx_gemm(qa, sa, qb, sb, out_dtype=torch.float32)), ref, absref, k, bf16=False)


def test_mx_gemm_full_fprop_sampled():
    """MXFP4 operands of the linear layer's fprop (X 16384 x 5120, W 20480 x
    5120): 16 sampled rows of the output against the oracle."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x_np, w_np, _ = wl.linear_layer()
    announce("mx full fprop 16384x20480x5120")
    qa, sa = nv.mx_quantize(to_device(x_np, "bf16"))
    qb, sb = nv.mx_quantize(to_device(w_np, "bf16"))
    c = nv.mx_gemm(qa, sa, qb, sb)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(8).choice(x_np.shape[0], 16, replace=False))
    rq, rs = o.mx_quantize(x_np[rows])
    idx = torch.as_tensor(rows, device="cuda")
    assert np.array_equal(host(qa[idx]), rq) and np.array_equal(host(sa[idx]), rs)
    ra = o.mx_dequantize(rq, rs).astype(np.float64)
    rb = o.mx_dequantize(host(qb), host(sb)).astype(np.float64)
    check(host(c[idx].float()), ra @ rb.T, np.abs(ra) @ np.abs(rb).T, x_np.shape[1])


def test_nvfp4_error_below_mxfp4_on_the_activation():
    """The pages' comparison (Resumen técnico §2): on the linear layer's
    activation, NVFP4's dequantization error is below MXFP4's."""
    require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x_np = wl.normal((2048, 5120), seed=5, outlier_channels=16, channel_gain=20.0)
    x = to_device(x_np, "bf16")
    q, s = nv.mx_quantize(x)
    err_mx = np.mean((host(nv.mx_dequantize(q, s)) - x_np) ** 2)
    row, _, _ = nv.quantize(x, outputs=nv.OUT_ROW)
    err_nv = np.mean((host(nv.dequantize(row)) - x_np) ** 2)
    announce(f"mse nvfp4 {err_nv:.4e} mxfp4 {err_mx:.4e}")
    assert err_nv < err_mx
