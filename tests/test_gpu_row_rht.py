"""GPU parity of nvfp4_quantize_row_rht, the one-read quantization of an
activation into its 1x16 row copy (round to nearest) and its Hadamard 16x1
column copy, each with its own tensor scale.

Criteria:
  (a) the row copy against the oracle's row quantization: bit for bit;
  (b) the Hadamard copy (codes, scale bytes, tensor scale and the transformed
      tensor's amax in amax_ws[1]) against the oracle:
        - bit for bit against the oracle quantizing the kernel's own
          transformed values (nvfp4_rht_transform), with the element indices
          of the stored transpose for SR;
        - end to end against the oracle's own transform: codes differ in at
          most 1e-5 of the elements and by at most one E2M1 step;
      at ragged shapes, RN and SR, bf16 and float32 inputs, and on sampled
      columns of the full-size activation of the linear layer;
  (c) every output of the fused call against separate nvfp4_quantize (1D, RN,
      row copy) and nvfp4_rht_quantize calls on the same input: bit for bit,
      including both amaxes and both tensor scales, also at full size.
"""

import numpy as np
import pytest

import oracle as o
import workloads as wl
from tests._helpers import announce, e2m1_step_distance, host, require_gpu, to_device

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


def _gpu_transform(x):
    """The kernel's own float32 transformed values of a device tensor x."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    out = torch.empty(tuple(x.shape), dtype=torch.float32, device="cuda")
    nv.nvfp4_rht_transform(x, wl.RHT_SEED, out)
    return host(out)


def _check_hadamard_copy(x_np, x, col, ws, rounding, seed, offset):
    """(b) for one fused call: the Hadamard copy `col` and amax_ws[1]."""
    rnd = "sr" if rounding == 1 else "rn"
    xt_gpu = _gpu_transform(x)
    # the transformed tensor's amax, bit for bit
    a = np.float32(np.max(np.abs(xt_gpu)))
    assert host(ws)[1] == a
    # bit for bit against the oracle quantizing the kernel's transformed values
    ref = o.quantize(xt_gpu, rounding=rnd, seed=seed, offset=offset, outputs=("col",))["col"]
    assert host(col.tensor_scale)[0] == ref.tensor_scale
    assert np.array_equal(host(col.scales), ref.scales)
    assert np.array_equal(host(col.codes), ref.codes)
    # end to end against the oracle's own (exactly rounded) transform
    e2e = o.rht_quantize(x_np, wl.RHT_SEED, rounding=rnd, seed=seed, offset=offset)
    d = e2m1_step_distance(o.unpack_codes(host(col.codes)), o.unpack_codes(e2e.codes))
    assert np.mean(d != 0) <= 1e-5, int(np.sum(d != 0))
    assert np.all(d <= 1)
    assert np.mean(host(col.scales) != e2e.scales) <= 1e-5
    assert abs(float(host(ws)[1]) - float(e2e.amax)) <= 1e-6 * float(e2e.amax)


@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("shape,dtype", [((16, 16), "bf16"), ((272, 400), "bf16"),
                                         ((528, 272), "bf16"), ((1040, 2064), "bf16"),
                                         ((2320, 400), "bf16"),
                                         ((272, 400), "fp32"), ((528, 144), "fp32")])
def test_hadamard_copy_against_oracle(shape, dtype, rounding):
    announce(f"row+rht hadamard copy vs oracle {shape} {dtype} r={rounding}")
    require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x_np = (wl.activation(shape[0], shape[1], seed=sum(shape)) if dtype == "bf16"
            else wl.normal(shape, 3, outlier_channels=2, dtype="fp32"))
    x = to_device(x_np, dtype)
    row, col, ws = nv.quantize_row_rht(x, wl.RHT_SEED, rounding_t=rounding, seed=11, offset=3)
    _check_hadamard_copy(x_np, x, col, ws, rounding, 11, 3)
    ref = o.quantize(x_np, outputs=("row",))["row"]
    assert np.array_equal(host(row.codes), ref.codes)
    assert np.array_equal(host(row.scales), ref.scales)
    assert host(ws)[0] == np.float32(np.max(np.abs(x_np)))


@pytest.mark.parametrize("rounding", [0, 1])
def test_full_activation_hadamard_copy_sampled(rounding):
    """The linear layer's activation X (16384 x 5120, bf16, 16 outlier
    channels), launched as in the training step: the transformed tensor's
    amax, and the Hadamard copy's scale bytes and codes on 32 sampled columns
    against the oracle quantizing the kernel's transformed values with the
    full tensor's element indices; the transformed values of those columns
    against the oracle's exact transform; the row copy on sampled rows."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    announce(f"row+rht full 16384x5120 hadamard copy vs oracle r={rounding}")
    x_np, _, _ = wl.linear_layer()
    t, h = x_np.shape
    x = to_device(x_np, "bf16")
    row, col, ws = nv.quantize_row_rht(x, wl.RHT_SEED, rounding_t=rounding, seed=wl.SR_SEED,
                                       offset=2)
    torch.cuda.synchronize()
    xt_full = o.rht(x_np, wl.RHT_SEED)
    a = np.float32(np.max(np.abs(xt_full)))
    assert abs(float(host(ws)[1]) - float(a)) <= 1e-6 * float(a)
    assert host(ws)[0] == np.float32(np.max(np.abs(x_np)))
    s_t = o.tensor_scale(host(ws)[1])
    assert host(col.tensor_scale)[0] == s_t
    cols = np.sort(np.random.default_rng(5).choice(h, 32, replace=False))
    xg = to_device(np.ascontiguousarray(x_np[:, cols]), "bf16")
    xt_gpu = _gpu_transform(xg)
    gb = xt_gpu.reshape(t // 16, 16, -1).astype(np.float64)
    wb = xt_full[:, cols].reshape(t // 16, 16, -1).astype(np.float64)
    bmax = np.max(np.abs(wb), axis=1, keepdims=True)
    assert np.all(np.abs(gb - wb) <= 1e-6 * bmax)
    rnd = "sr" if rounding == 1 else "rn"
    sub = np.ascontiguousarray(xt_gpu.T)
    for i, c in enumerate(cols):
        codes, sb = o.quantize_rows(sub[i:i + 1], s_t, rnd, seed=wl.SR_SEED, offset=2, stream=1,
                                    index_base=int(c) * t)
        assert np.array_equal(host(col.scales[c:c + 1]), sb), int(c)
        assert np.array_equal(host(col.codes[c:c + 1]), o.pack_codes(codes)), int(c)
    rows = np.sort(np.random.default_rng(6).choice(t, 64, replace=False))
    s_row = o.tensor_scale(np.float32(np.max(np.abs(x_np))))
    assert host(row.tensor_scale)[0] == s_row
    codes, sb = o.quantize_rows(x_np[rows], s_row, "rn")
    assert np.array_equal(host(row.codes)[rows], o.pack_codes(codes))
    assert np.array_equal(host(row.scales)[rows], sb)
