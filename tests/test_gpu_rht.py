"""GPU parity of the weight-gradient operand path (16-point random Hadamard
transform along tokens + 16x1 NVFP4, RN or SR) and of the Philox words.

The comparison is split so each part has its own exact criterion:
  (a) Philox words: bit for bit;
  (b) transformed values: within 1e-6 of the 16-block's largest magnitude
      (float32 butterfly vs the oracle's exactly rounded dense product);
  (c) quantization of the GPU's own transformed values: bit for bit;
  (d) end to end against the oracle from scratch: codes differ in at most
      1e-5 of the elements and by at most one E2M1 step.
"""

import numpy as np
import pytest

import oracle as o
import workloads as wl
from tests._helpers import announce, e2m1_step_distance, host, require_gpu, to_device

pytestmark = pytest.mark.gpu


def test_philox_words_bit_exact():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    for seed, c2, c3, n in ((7, 0, 1, 4096), ((1 << 40) + 5, 0xFFFFFFFF, 0, 1000), (0, 3, 2, 17)):
        out = torch.empty(4 * n, dtype=torch.int32, device="cuda")
        nv.nvfp4_philox_fill(seed, c2, c3, n, out)
        got = host(out).view(np.uint32).reshape(n, 4)
        g = np.arange(n, dtype=np.uint64)
        ctr = np.stack([g & 0xFFFFFFFF, g >> 32, np.full_like(g, c2), np.full_like(g, c3)], -1)
        want = o.philox4x32_10((seed & 0xFFFFFFFF, seed >> 32), ctr)
        assert np.array_equal(got, want)


def gpu_transform(x_np, dtype, seed):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x = to_device(x_np, dtype)
    out = torch.empty(x_np.shape, dtype=torch.float32, device="cuda")
    nv.nvfp4_rht_transform(x, seed, out)
    return host(out)


def assert_transform_close(got, want):
    t, c = want.shape
    gb = got.reshape(t // 16, 16, c).astype(np.float64)
    wb = want.reshape(t // 16, 16, c).astype(np.float64)
    bmax = np.max(np.abs(wb), axis=1, keepdims=True)
    err = np.abs(gb - wb)
    assert np.all(err <= 1e-6 * bmax), float(np.max(err / np.maximum(bmax, 1e-30)))


@pytest.mark.parametrize("shape,dtype", [((16, 16), "bf16"), ((272, 400), "bf16"),
                                         ((528, 144), "fp32")])
def test_transform_values(shape, dtype):
    announce(f"rht transform {shape} {dtype}")
    x = wl.laplace(shape, seed=1, dtype=dtype) if dtype == "bf16" else wl.normal(shape, 2, dtype="fp32")
    got = gpu_transform(x, dtype, 7)
    assert_transform_close(got, o.rht(x, 7))


def run_rht_quantize(x_np, dtype, rounding, seed=7, offset=0, rht_seed=7):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x = to_device(x_np, dtype)
    q, ws = nv.rht_quantize(x, rht_seed, rounding=rounding, seed=seed, offset=offset)
    torch.cuda.synchronize()
    return q, ws


@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("shape", [(16, 32), (272, 400), (528, 272)])
def test_quantization_of_transformed_values_bit_exact(shape, rounding):
    announce(f"rht quantize {shape} r={rounding}")
    x = wl.laplace(shape, seed=3)
    q, ws = run_rht_quantize(x, "bf16", rounding, seed=7, offset=5)
    xt_gpu = gpu_transform(x, "bf16", 7)
    a = np.float32(np.max(np.abs(xt_gpu)))
    assert host(ws)[0] == a
    ref = o.quantize(xt_gpu, rounding="rn" if rounding == 0 else "sr", seed=7, offset=5,
                     outputs=("col",))["col"]
    assert host(q.tensor_scale)[0] == ref.tensor_scale
    assert np.array_equal(host(q.scales), ref.scales)
    assert np.array_equal(host(q.codes), ref.codes)


@pytest.mark.parametrize("k", [-70, -55, 0, 60])
def test_quantization_bit_exact_across_tensor_scales(k):
    """bf16 input scaled by 2^k: the transform scales exactly, and the block
    scales (reciprocal and correction step, or IEEE division for tiny tensor
    scales) must still equal the oracle's on the kernel's transformed values."""
    announce(f"rht quantize scaled 2^{k}")
    x = wl.to_bf16_values(wl.activation(272, 400, seed=12) * np.float32(2.0 ** k))
    for rounding in (0, 1):
        q, ws = run_rht_quantize(x, "bf16", rounding, seed=7, offset=2)
        xt_gpu = gpu_transform(x, "bf16", 7)
        assert host(ws)[0] == np.float32(np.max(np.abs(xt_gpu)))
        ref = o.quantize(xt_gpu, rounding="rn" if rounding == 0 else "sr", seed=7, offset=2,
                         outputs=("col",))["col"]
        assert host(q.tensor_scale)[0] == ref.tensor_scale
        assert np.array_equal(host(q.scales), ref.scales)
        assert np.array_equal(host(q.codes), ref.codes)


@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_end_to_end_against_oracle(rounding):
    x = wl.laplace((1024, 512), seed=8)
    announce(f"rht end-to-end {rounding}")
    q, _ = run_rht_quantize(x, "bf16", 0 if rounding == "rn" else 1, seed=7, offset=0)
    ref = o.rht_quantize(x, 7, rounding=rounding, seed=7, offset=0)
    got = o.unpack_codes(host(q.codes))
    want = o.unpack_codes(ref.codes)
    d = e2m1_step_distance(got, want)
    assert np.mean(d != 0) <= 1e-5
    assert np.all(d <= 1)
    sb_diff = np.mean(host(q.scales) != ref.scales)
    assert sb_diff <= 1e-5


def _full_rht_sampled(x, rounding, seed):
    """RHT (seed 7) + RN or SR (Philox seed `seed`) of a full-size bf16 tensor:
    the tensor amax, the transformed values of 32 sampled columns, and their
    scale bytes and codes (the oracle quantizing the kernel's own transformed
    values, with the element indices of the full tensor)."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    q, ws = run_rht_quantize(x, "bf16", 1 if rounding == "sr" else 0, seed=seed, offset=0,
                             rht_seed=wl.RHT_SEED)
    xt_full = o.rht(x, wl.RHT_SEED)
    a = np.float32(np.max(np.abs(xt_full)))
    assert abs(float(host(ws)[0]) - float(a)) <= 1e-6 * float(a)
    s = o.tensor_scale(host(ws)[0])
    cols = np.sort(np.random.default_rng(2).choice(x.shape[1], 32, replace=False))
    # GPU transform of the sampled columns (same kernel, contiguous slice copy)
    xg = to_device(np.ascontiguousarray(x[:, cols]), "bf16")
    out = torch.empty(xg.shape, dtype=torch.float32, device="cuda")
    nv.nvfp4_rht_transform(xg, wl.RHT_SEED, out)
    xt_gpu = host(out)
    assert_transform_close(xt_gpu, xt_full[:, cols])
    t = x.shape[0]
    sub = np.ascontiguousarray(xt_gpu.T)  # [32, T]
    for i, c in enumerate(cols):
        codes, sb = o.quantize_rows(sub[i:i + 1], s, rounding, seed=seed, offset=0, stream=1,
                                    index_base=int(c) * t)
        assert np.array_equal(host(q.scales[c:c + 1]), sb), int(c)
        assert np.array_equal(host(q.codes[c:c + 1]), o.pack_codes(codes)), int(c)


def test_full_gradient_sr_sampled():
    """bf16 dY 8192x20480 Laplace(0, 1e-3), RHT (seed 7) + SR (Philox seed 7):
    transformed values and codes checked on sampled columns."""
    announce("full gradient 8192x20480 RHT+SR")
    _full_rht_sampled(wl.gradient(), "sr", wl.SR_SEED)


@pytest.mark.parametrize("rounding", ["rn", "sr"])
def test_full_wgrad_activation_sampled(rounding):
    """The other weight-gradient operand: bf16 X 8192x5120 N(0,1), RHT with
    the same signs, RN (the recipe's choice for activations) and SR."""
    announce(f"full wgrad activation 8192x5120 RHT+{rounding}")
    _full_rht_sampled(wl.wgrad_activation(), rounding, wl.SR_SEED)
