"""GPU parity of the dgrad path of the linear layer: dY quantized row-wise in
1x16 blocks with stochastic rounding (its row copy, Philox stream 0), then
dX = deq(Q_SR(dY)) . deq(Q2D(W)), whose B operand is the transposed 16x16
copy of W (W^T codes and the transposed grid, K = ffn contiguous), the copy
the weight quantizer writes beside W's own.

Source: gist.science summary of "Pretraining Large Language Models with
NVFP4", Resumen técnico §2 "Precisión Mixta Selectiva" (the three GEMMs of a
linear layer, dgrad among them, run on NVFP4 operands) and "Escalado
Bidimensional (2D) y Redondeo Estocástico" (16x16 weight blocks so that W
and W^T quantize identically; stochastic rounding of gradients).

Criteria: the quantized dY matches the oracle bit for bit; the GEMM meets the
bound of the other GEMM tests (relative Frobenius error <= 1e-2 against the
oracle's dequantize-then-matmul, plus the per-element bound).
"""

import numpy as np
import pytest

import oracle as o
import workloads as wl
from tests._helpers import announce, host, require_gpu, to_device
from tests.test_gpu_gemm import check

pytestmark = pytest.mark.gpu


def dgrad_operands(t, f, h, seed):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    dy = wl.laplace((t, f), seed=seed)
    w = wl.weight(f, h, seed=seed + 1)
    a, _, _ = nv.quantize(to_device(dy, "bf16"), rounding=nv.ROUND_SR, seed=wl.SR_SEED,
                          offset=seed, outputs=nv.OUT_ROW)
    w_row, w_col, _ = nv.quantize(to_device(w, "bf16"), block=nv.BLOCK_2D,
                                  outputs=nv.OUT_ROW | nv.OUT_COL)
    torch.cuda.synchronize()
    return dy, w, a, w_row, w_col


@pytest.mark.parametrize("t,f,h", [(256, 512, 256), (300, 784, 272), (1024, 2048, 512)])
def test_dgrad_parity(t, f, h):
    import bit_block_scaled_bf16_amd as nv

    announce(f"dgrad {t}x{h}x{f}")
    dy, w, a, w_row, w_col = dgrad_operands(t, f, h, seed=t + f)
    # the SR row copy of dY, bit for bit
    ref = o.quantize(dy, rounding="sr", seed=wl.SR_SEED, offset=t + f, outputs=("row",))["row"]
    assert np.array_equal(host(a.codes), ref.codes)
    assert np.array_equal(host(a.scales), ref.scales)
    # W^T's copy dequantizes to exactly the transpose of W's
    dw = o.dequantize(host(w_row.codes), host(w_row.scales), host(w_row.tensor_scale)[0], "2d")
    dwt = o.dequantize(host(w_col.codes), host(w_col.scales), host(w_col.tensor_scale)[0], "2d")
    assert np.array_equal(dw.T, dwt)
    # dX [t, h] = deq(Q_SR(dY)) deq(W)
    dx = host(nv.gemm(a, w_col).float())
    ra = o.dequantize(host(a.codes), host(a.scales), host(a.tensor_scale)[0], "1d").astype(np.float64)
    rb = dwt.astype(np.float64)
    check(dx, ra @ rb.T, np.abs(ra) @ np.abs(rb).T, f)


def test_full_dgrad_sampled():
    """dX = deq(Q_SR(dY)) deq(Q2D(W)) at the linear-layer shape: dY 16384 x
    20480, W 20480 x 5120, bf16 dX 16384 x 5120. 16 sampled rows of the SR
    row copy (bit for bit, with the element indices of the full tensor) and
    the same rows of dX are checked."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x_np, w_np, dy_np = wl.linear_layer()
    del x_np
    announce("full dgrad 16384x5120x20480")
    a, _, ws = nv.quantize(to_device(dy_np, "bf16"), rounding=nv.ROUND_SR, seed=wl.SR_SEED,
                           offset=0, outputs=nv.OUT_ROW)
    _, w_col, _ = nv.quantize(to_device(w_np, "bf16"), block=nv.BLOCK_2D, outputs=nv.OUT_COL)
    dx = nv.gemm(a, w_col)
    torch.cuda.synchronize()
    amax = np.float32(np.max(np.abs(dy_np)))
    assert host(ws)[0] == amax
    s = o.tensor_scale(amax)
    f = dy_np.shape[1]
    rows = np.sort(np.random.default_rng(7).choice(dy_np.shape[0], 16, replace=False))
    for r in rows:
        codes, sb = o.quantize_rows(dy_np[r:r + 1], s, "sr", seed=wl.SR_SEED, offset=0, stream=0,
                                    index_base=int(r) * f)
        assert np.array_equal(host(a.codes[r:r + 1]), o.pack_codes(codes)), int(r)
        assert np.array_equal(host(a.scales[r:r + 1]), sb), int(r)
    idx = torch.as_tensor(rows, device="cuda")
    ra = o.dequantize(host(a.codes[idx]), host(a.scales[idx]), host(a.tensor_scale)[0],
                      "1d").astype(np.float64)
    rb = o.dequantize(host(w_col.codes), host(w_col.scales), host(w_col.tensor_scale)[0],
                      "2d").astype(np.float64)
    check(host(dx[idx].float()), ra @ rb.T, np.abs(ra) @ np.abs(rb).T, f)
