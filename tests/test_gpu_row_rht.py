"""GPU parity of nvfp4_quantize_row_rht, the one-read quantization of an
activation into its 1x16 row copy (round to nearest) and its Hadamard 16x1
column copy, each with its own tensor scale.

Criteria:
  (a) the row copy against the oracle's row quantization: bit for bit;
  (b) every output of the fused call against separate nvfp4_quantize (1D, RN,
      row copy) and nvfp4_rht_quantize calls on the same input: bit for bit
      (the separate calls carry their own oracle parity in the quantize and
      RHT tests), including both amaxes and both tensor scales;
  (c) the full-size activation of the linear layer, launched as in the
      training step: (b) on every byte.
"""

import numpy as np
import pytest

import oracle as o
import workloads as wl
from tests._helpers import announce, host, require_gpu, to_device

pytestmark = pytest.mark.gpu


def fused_and_separate(x, rounding, seed=7, offset=0, rht_seed=7, amax=None):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    row, col, ws = nv.quantize_row_rht(x, rht_seed, rounding_t=rounding, seed=seed, offset=offset,
                                       amax=amax)
    amax_row = amax_t = None
    if amax is not None:
        # the library wants 16-byte aligned amax pointers: one tensor each
        amax_row = torch.zeros(4, dtype=torch.float32, device=amax.device)
        amax_t = torch.zeros(4, dtype=torch.float32, device=amax.device)
        amax_row[0], amax_t[0] = amax[0], amax[1]
    row_ref, _, ws_row = nv.quantize(x, outputs=nv.OUT_ROW, amax=amax_row)
    col_ref, ws_t = nv.rht_quantize(x, rht_seed, rounding=rounding, seed=seed, offset=offset,
                                    amax=amax_t)
    torch.cuda.synchronize()
    return (row, col, ws), (row_ref, col_ref, ws_row, ws_t)


def assert_same(fused, separate, amax_given=False):
    row, col, ws = fused
    row_ref, col_ref, ws_row, ws_t = separate
    for got, want in ((row, row_ref), (col, col_ref)):
        assert np.array_equal(host(got.codes), host(want.codes))
        assert np.array_equal(host(got.scales), host(want.scales))
        assert host(got.tensor_scale)[0] == host(want.tensor_scale)[0]
    if not amax_given:
        w = host(ws)
        assert w[0] == host(ws_row)[0] and w[1] == host(ws_t)[0]


@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("shape,dtype", [((16, 16), "bf16"), ((272, 400), "bf16"),
                                         ((528, 272), "bf16"), ((1040, 2064), "bf16"),
                                         ((272, 400), "fp32"), ((528, 144), "fp32")])
def test_fused_equals_separate_calls(shape, dtype, rounding):
    announce(f"row+rht {shape} {dtype} r={rounding}")
    x_np = wl.laplace(shape, seed=sum(shape)) if dtype == "bf16" else wl.normal(shape, 2, dtype="fp32")
    x = to_device(x_np, dtype)
    fused, separate = fused_and_separate(x, rounding, seed=11, offset=3)
    assert_same(fused, separate)


def test_row_copy_against_oracle():
    announce("row+rht row copy vs oracle")
    require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x_np = wl.activation(528, 400, seed=4)
    row, _, ws = nv.quantize_row_rht(to_device(x_np, "bf16"), 7)
    ref = o.quantize(x_np, outputs=("row",))["row"]
    assert np.array_equal(host(row.codes), ref.codes)
    assert np.array_equal(host(row.scales), ref.scales)
    assert host(row.tensor_scale)[0] == ref.tensor_scale
    assert host(ws)[0] == np.float32(np.max(np.abs(x_np)))


def test_amax_given():
    torch = require_gpu()

    announce("row+rht amax_in")
    x_np = wl.laplace((272, 400), seed=9)
    x = to_device(x_np, "bf16")
    # larger than both true amaxes: the two tensor scales differ from the
    # computed ones and from each other
    amax = torch.tensor([50.0, 70.0, 0.0, 0.0], dtype=torch.float32, device="cuda")
    fused, separate = fused_and_separate(x, 1, seed=5, amax=amax)
    assert_same(fused, separate, amax_given=True)
    assert host(fused[0].tensor_scale)[0] == o.tensor_scale(np.float32(50.0))
    assert host(fused[1].tensor_scale)[0] == o.tensor_scale(np.float32(70.0))


def test_empty_tensor():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    announce("row+rht empty")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    row, col, ws = nv.quantize_row_rht(x, 7)
    torch.cuda.synchronize()
    assert host(row.tensor_scale)[0] == 1.0 and host(col.tensor_scale)[0] == 1.0
    assert host(ws)[0] == 0.0 and host(ws)[1] == 0.0


def test_full_activation_equals_separate_calls():
    """The linear layer's activation X (16384 x 5120, bf16), RN column copy as
    in the training step: every byte of both copies."""
    announce("row+rht full 16384x5120")
    x_np, _, _ = wl.linear_layer()
    x = to_device(x_np, "bf16")
    fused, separate = fused_and_separate(x, 0, rht_seed=wl.RHT_SEED)
    assert_same(fused, separate)
