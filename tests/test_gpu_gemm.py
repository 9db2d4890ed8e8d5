"""GPU parity of nvfp4_gemm with the oracle's dequantize-then-matmul.

Criterion (stated bar): relative Frobenius error <= 1e-2 against the oracle's
float32 dequantization multiplied in float64. A tighter per-element bound is
checked too: the GPU differs from the exact product only by float32
accumulation (each product is exact) and the final rounding to bf16, so
|C - C_ref| <= 2^-8 |C_ref| + K 2^-23 (|A| |B|^T).
"""

import numpy as np
import pytest

import oracle as o
import workloads as wl
from tests._helpers import announce, host, require_gpu, to_device

pytestmark = pytest.mark.gpu


def quantized_operands(m, n, k, b_2d=False, seed=0):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    a_np = wl.activation(m, k, seed=seed) if k >= 256 else wl.normal((m, k), seed=seed)
    if b_2d:
        b_np = wl.weight(n, k, seed=seed + 1)
        b, _, _ = nv.quantize(to_device(b_np, "bf16"), block=nv.BLOCK_2D, outputs=nv.OUT_ROW)
    else:
        b_np = wl.normal((n, k), seed=seed + 1)
        b, _, _ = nv.quantize(to_device(b_np, "bf16"), outputs=nv.OUT_ROW)
    a, _, _ = nv.quantize(to_device(a_np, "bf16"), outputs=nv.OUT_ROW)
    torch.cuda.synchronize()
    return a, b


def reference(a, b):
    ra = o.dequantize(host(a.codes), host(a.scales), host(a.tensor_scale)[0],
                      "2d" if a.block == 1 else "1d").astype(np.float64)
    rb = o.dequantize(host(b.codes), host(b.scales), host(b.tensor_scale)[0],
                      "2d" if b.block == 1 else "1d").astype(np.float64)
    return ra @ rb.T, np.abs(ra) @ np.abs(rb).T


def check(c_gpu, ref, absref, k, bf16=True):
    c = c_gpu.astype(np.float64)
    fro = np.linalg.norm(c - ref) / max(np.linalg.norm(ref), 1e-30)
    assert fro <= 1e-2, fro
    rel = 2.0 ** -8 if bf16 else 2.0 ** -22
    bound = rel * np.abs(ref) + k * 2.0 ** -23 * absref + 1e-30
    assert np.all(np.abs(c - ref) <= bound), float(np.max(np.abs(c - ref) / bound))
    return fro


# Shapes up to a quarter of the CUs' worth of 256 x 256 tiles run entirely as
# 128 x 128 tiles; (2500, 2600, 208) runs entirely as 256 x 256 tiles with
# ragged edges and a ragged K; (4100 | 4312, 4080, *) give 272 tiles, i.e. one
# full round of 256 x 256 tiles plus a last round of 128 x 128 quarters on
# 256 CUs, including quarters partly or wholly past the ragged edges.
# Several rounds of whole 256 x 256 tiles: (4096, 8192, 256) gives 512 tiles,
# two full rounds; (4352, 8192, 384) two full rounds plus a last round of 32
# tiles as quarters; (1024, 22784, 256) 356 tiles, a full round and a last
# round of 100 tiles, too many for quarters.
# Tile blocks per XCD (tile_of): (4096, 8192, 256) is 16 x 32 tiles, sixteen
# 4 x 8 blocks; (3072, 6144, 256) 12 x 24 tiles, nine 4 x 8 blocks, the last
# in plain order and run as quarters; (4096, 5120, 256) 16 x 20 tiles, ten
# 8 x 4 blocks, the last two in plain order and run as quarters.
@pytest.mark.parametrize("m,n,k", [(16, 16, 16), (256, 256, 64), (300, 520, 80), (512, 768, 1024),
                                   (33, 47, 208), (272, 256, 5120), (2500, 2608, 208),
                                   (4312, 4080, 336), (4100, 4080, 384), (4096, 8192, 256),
                                   (4352, 8192, 384), (1024, 22784, 256), (3072, 6144, 256),
                                   (4096, 5120, 256)])
@pytest.mark.parametrize("b_2d", [False, True])
def test_gemm_parity(m, n, k, b_2d):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    announce(f"gemm {m}x{n}x{k} b2d={b_2d}")
    if b_2d and n % 16:
        # 16x16 blocks need N % 16 == 0: the call is refused before any launch
        a, _ = quantized_operands(m, 16, k, False, seed=m + n + k)
        qb = torch.zeros((n, k // 2), dtype=torch.uint8, device="cuda")
        sb = torch.zeros(((n + 15) // 16, k // 16), dtype=torch.uint8, device="cuda")
        c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(nv.Nvfp4Error) as err:
            nv.nvfp4_gemm(a.codes, a.scales, a.tensor_scale, nv.BLOCK_1D, qb, sb, a.tensor_scale,
                          nv.BLOCK_2D, m, n, k, c)
        assert err.value.status == nv._lib.ERR_SHAPE
        return
    a, b = quantized_operands(m, n, k, b_2d, seed=m + n + k)
    ref, absref = reference(a, b)
    c = host(nv.gemm(a, b).float())
    check(c, ref, absref, k)
    c32 = host(nv.gemm(a, b, out_dtype=torch.float32))
    check(c32, ref, absref, k, bf16=False)


def test_gemm_all_ones_closed_form():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    m, n, k = 64, 96, 4096
    # operands built directly: code 0x2 (1.0), scale 0x38 (1.0), S = 1
    qa = torch.full((m, k // 2), 0x22, dtype=torch.uint8, device="cuda")
    sa = torch.full((m, k // 16), 0x38, dtype=torch.uint8, device="cuda")
    qb = torch.full((n, k // 2), 0x22, dtype=torch.uint8, device="cuda")
    sb = torch.full((n // 16, k // 16), 0x38, dtype=torch.uint8, device="cuda")
    one = torch.tensor([1.0, 0, 0, 0], dtype=torch.float32, device="cuda")
    c = torch.empty((m, n), dtype=torch.float32, device="cuda")
    nv.nvfp4_gemm(qa, sa, one, nv.BLOCK_1D, qb, sb, one, nv.BLOCK_2D, m, n, k, c)
    assert np.all(host(c) == float(k))


def test_gemm_bf16_output_rounds_to_nearest_even():
    """C = 1 + 2^-8 and 1 + 3 * 2^-8 are exact float32 sums that sit halfway
    between bf16 neighbours; round to nearest even gives 1.0 and 1.015625."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    k = 32
    # row 0: block 0 = one 1.0 (code 0x2, scale 0x38); block 1 = one 0.5 (code
    # 0x1) at scale 2^-7 (0x04) -> 2^-8. row 1: same with 3 * 0.5 * 2^-7.
    qa = torch.zeros((2, k // 2), dtype=torch.uint8, device="cuda")
    qa[0, 0] = 0x02
    qa[0, 8] = 0x01
    qa[1, 0] = 0x02
    qa[1, 8] = 0x11  # two 0.5 values
    qa[1, 9] = 0x01  # a third 0.5
    sa = torch.tensor([[0x38, 0x04], [0x38, 0x04]], dtype=torch.uint8, device="cuda")
    qb = torch.full((16, k // 2), 0x22, dtype=torch.uint8, device="cuda")  # all 1.0
    sb = torch.full((16, k // 16), 0x38, dtype=torch.uint8, device="cuda")
    one = torch.tensor([1.0, 0, 0, 0], dtype=torch.float32, device="cuda")
    c = torch.empty((2, 16), dtype=torch.bfloat16, device="cuda")
    nv.nvfp4_gemm(qa, sa, one, nv.BLOCK_1D, qb, sb, one, nv.BLOCK_1D, 2, 16, k, c)
    got = host(c.float())
    assert np.all(got[0] == 1.0) and np.all(got[1] == 1.015625)
    c32 = torch.empty((2, 16), dtype=torch.float32, device="cuda")
    nv.nvfp4_gemm(qa, sa, one, nv.BLOCK_1D, qb, sb, one, nv.BLOCK_1D, 2, 16, k, c32)
    got32 = host(c32)
    assert np.all(got32[0] == 1.0 + 2.0 ** -8) and np.all(got32[1] == 1.0 + 3 * 2.0 ** -8)


def test_gemm_empty_k_writes_zeros():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    one = torch.tensor([1.0, 0, 0, 0], dtype=torch.float32, device="cuda")
    c = torch.full((40, 24), 7.0, dtype=torch.float32, device="cuda")
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    nv.nvfp4_gemm(dummy, dummy, one, 0, dummy, dummy, one, 0, 40, 24, 0, c)
    assert np.all(host(c) == 0.0)


def test_gemm_ldc():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    a, b = quantized_operands(128, 200, 256, seed=3)
    ref, absref = reference(a, b)
    big = torch.zeros((128, 264), dtype=torch.bfloat16, device="cuda")
    nv.gemm(a, b, out=big[:, 8:208])
    got = host(big.float())
    check(got[:, 8:208], ref, absref, 256)
    assert np.all(got[:, :8] == 0) and np.all(got[:, 208:] == 0)


# ---------------------------------------------------------------------------
# Full-size linear layer, checked on sampled rows and columns of C.
# ---------------------------------------------------------------------------


def _sampled_check(a, b, c, rows, cols, k):
    import torch

    idx = torch.as_tensor(rows, device=a.codes.device)
    qa, sa = host(a.codes[idx]), host(a.scales[idx])
    ra = o.dequantize(qa, sa, host(a.tensor_scale)[0], "1d").astype(np.float64)
    rb_all_codes, rb_all_scales = host(b.codes), host(b.scales)
    rb = o.dequantize(rb_all_codes, rb_all_scales, host(b.tensor_scale)[0],
                      "2d" if b.block == 1 else "1d").astype(np.float64)
    ref = ra @ rb.T
    absref = np.abs(ra) @ np.abs(rb).T
    check(host(c[idx].float()), ref, absref, k)
    return ref


def test_full_fprop_sampled():
    """Y = deq(Q(X)) deq(Q2D(W))^T, X 16384x5120, W 20480x5120, bf16 out;
    16 sampled rows of Y (all 20480 columns) checked against the oracle."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x_np, w_np, _ = wl.linear_layer()
    announce("full fprop 16384x20480x5120")
    a, _, _ = nv.quantize(to_device(x_np, "bf16"), outputs=nv.OUT_ROW)
    b, _, _ = nv.quantize(to_device(w_np, "bf16"), block=nv.BLOCK_2D, outputs=nv.OUT_ROW)
    c = nv.gemm(a, b)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(x_np.shape[0], 16, replace=False))
    _sampled_check(a, b, c, rows, None, x_np.shape[1])


def test_full_wgrad_sampled():
    """dW = deq(Q_SR(RHT(dY)))^T-copy . deq(Q(RHT(X)))^T-copy: A [20480, 16384],
    B [5120, 16384], bf16 out; 16 sampled rows of dW checked."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x_np, _, dy_np = wl.linear_layer()
    announce("full wgrad 20480x5120x16384")
    a, _ = nv.rht_quantize(to_device(dy_np, "bf16"), wl.RHT_SEED, rounding=nv.ROUND_SR,
                           seed=wl.SR_SEED)
    b, _ = nv.rht_quantize(to_device(x_np, "bf16"), wl.RHT_SEED, rounding=nv.ROUND_RN)
    c = nv.gemm(a, b)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(6).choice(a.rows, 16, replace=False))
    _sampled_check(a, b, c, rows, None, a.cols)
