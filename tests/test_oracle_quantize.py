"""Pins of the oracle's scale chain, layouts, stochastic rounding and dequant.

* Hand-worked blocks (tests/golden/worked_blocks.json): every expected byte and
  value derived by hand from the format definitions.
* Power-of-two invariance: scaling a tensor by 2^k leaves every code and scale
  byte unchanged and scales S by 2^k exactly.
* Block-max invariant: in a block whose scale byte is a normal E4M3 number the
  element of largest magnitude always gets magnitude code 7 (value 6).
* Orientation identities: the column copy is the row copy of the transpose;
  the 16x16 weight codes of W^T are the transposed codes of W, so W and W^T
  dequantize to transposes of each other bit for bit.
* Stochastic rounding: over all 2^16 random words, the number that round up is
  exactly floor(frac * 2^16), and they are the largest words; the mean of
  many SR draws equals the input within a stated sigma bound.
* Memory: 0.5 + 1/16 bytes per element (4.5 bits), 1.78x smaller than FP8.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle as o

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_blocks.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_row_blocks(golden):
    case = golden["row_case"]
    x = np.concatenate([np.array(b["values"], dtype=np.float32) for b in case["blocks"]])[None, :]
    q = o.quantize(x, outputs=("row",))["row"]
    assert q.tensor_scale == np.float32(case["tensor_scale"])
    assert [int(v) for v in q.scales[0]] == [int(b["scale"], 16) for b in case["blocks"]]
    codes = o.unpack_codes(q.codes)[0]
    assert codes.tolist() == sum((b["codes"] for b in case["blocks"]), [])
    deq = o.dequantize(q.codes, q.scales, q.tensor_scale)[0]
    want = np.array(sum((b["dequant"] for b in case["blocks"]), []), dtype=np.float32)
    assert np.array_equal(deq, want)
    assert np.array_equal(np.signbit(deq), np.signbit(want))


def _tile_tensor(case):
    x = np.zeros(case["shape"], dtype=np.float32)
    for f in case["fill"]:
        ti, tj = f["tile"]
        x[16 * ti:16 * ti + 16, 16 * tj:16 * tj + 16] = f["value"]
        for r, c, v in f["set"]:
            x[r, c] = v
    return x


def test_golden_tile(golden):
    case = golden["tile_case"]
    x = _tile_tensor(case)
    q = o.quantize_2d(x)
    assert q["row"].tensor_scale == np.float32(case["tensor_scale"])
    grid = np.array([[int(v, 16) for v in row] for row in case["grid"]], dtype=np.uint8)
    assert np.array_equal(q["row"].scales, grid)
    assert np.array_equal(q["col"].scales, grid.T)
    codes = o.unpack_codes(q["row"].codes)
    lut = {float(k): v for k, v in case["codes_by_value"].items()}
    want = np.vectorize(lambda v: lut[float(v)])(x)
    assert np.array_equal(codes, want)


def _sample_tensor(shape, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        idx = rng.choice(x.size, max(1, x.size // 1000), replace=False)
        x.reshape(-1)[idx] *= 50
    return x


@pytest.mark.parametrize("k", [-20, -3, 1, 7, 30])
def test_power_of_two_invariance(k):
    x = _sample_tensor((64, 128), 0)
    a = o.quantize(x)
    b = o.quantize((x * np.float32(2.0 ** k)).astype(np.float32))
    for side in ("row", "col"):
        assert np.array_equal(a[side].codes, b[side].codes)
        assert np.array_equal(a[side].scales, b[side].scales)
    assert b["row"].tensor_scale == np.float32(a["row"].tensor_scale * np.float32(2.0 ** k))
    a2, b2 = o.quantize_2d(x), o.quantize_2d((x * np.float32(2.0 ** k)).astype(np.float32))
    assert np.array_equal(a2["row"].codes, b2["row"].codes)
    assert np.array_equal(a2["row"].scales, b2["row"].scales)


def test_block_max_maps_to_largest_code():
    x = _sample_tensor((128, 256), 1)
    q = o.quantize(x, outputs=("row",))["row"]
    codes = o.unpack_codes(q.codes).reshape(128, 16, 16)
    blocks = x.reshape(128, 16, 16)
    arg = np.argmax(np.abs(blocks), axis=2)
    top = np.take_along_axis(codes, arg[:, :, None], axis=2)[:, :, 0] & 7
    normal = q.scales >= 0x08
    assert normal.any()
    assert np.all(top[normal] == 7)


def test_tensor_scale_definition():
    assert o.tensor_scale(np.float32(2688.0)) == np.float32(1.0)
    assert o.tensor_scale(np.float32(0.0)) == np.float32(1.0)
    assert o.tensor_scale(np.float32(1e-30)) == np.float32(1.0)  # below 2^-100 * 2688
    assert o.tensor_scale(np.float32(5376.0)) == np.float32(2.0)
    with pytest.raises(ValueError):
        o.tensor_scale(np.float32(np.inf))


def test_zero_and_vanishing_tensors_quantize_to_zero():
    for v in (0.0, -0.0, 1e-31):
        x = np.full((16, 32), v, dtype=np.float32)
        q = o.quantize(x)
        for side in ("row", "col"):
            assert not q[side].codes.any() and not q[side].scales.any()
            assert q[side].tensor_scale == np.float32(1.0)


def test_non_finite_input_raises():
    x = np.zeros((16, 16), dtype=np.float32)
    x[3, 4] = np.nan
    with pytest.raises(ValueError):
        o.quantize(x)


def test_column_copy_is_row_copy_of_transpose():
    x = _sample_tensor((48, 80), 2)
    q = o.quantize(x)
    qt = o.quantize(np.ascontiguousarray(x.T), outputs=("row",))
    assert np.array_equal(q["col"].codes, qt["row"].codes)
    assert np.array_equal(q["col"].scales, qt["row"].scales)
    assert q["col"].tensor_scale == q["row"].tensor_scale


def test_2d_weights_identical_in_both_directions():
    # Resumen tecnico §2 "Escalado Bidimensional": the same quantized weights
    # serve the forward and the backward pass.
    w = (0.02 * np.random.default_rng(3).standard_normal((64, 96))).astype(np.float32)
    q = o.quantize_2d(w)
    qt = o.quantize_2d(np.ascontiguousarray(w.T))
    assert np.array_equal(q["col"].codes, qt["row"].codes)
    assert np.array_equal(q["col"].scales, qt["row"].scales)
    d = o.dequantize(q["row"].codes, q["row"].scales, q["row"].tensor_scale, "2d")
    dt = o.dequantize(q["col"].codes, q["col"].scales, q["col"].tensor_scale, "2d")
    assert np.array_equal(d.T, dt)


def test_dequant_error_is_bounded():
    x = _sample_tensor((64, 64), 4, outliers=False)
    q = o.quantize(x, outputs=("row",))["row"]
    d = o.dequantize(q.codes, q.scales, q.tensor_scale)
    # per block: error <= half the largest E2M1 gap (1) times s_f * S, plus
    # the saturation of the block max (y <= 6 * (1 + 2^-4))
    sf = np.repeat(o.e4m3_decode(q.scales), 16, axis=1) * q.tensor_scale
    assert np.all(np.abs(d - x) <= sf * 1.0 + 1e-12)


@pytest.mark.parametrize("y", [0.1, 0.3, 0.5, 0.7, 1.1, 1.2345, 2.2, 3.3, 4.5, 5.9, 6.0, 7.5, 2.0 ** -20])
def test_sr_counts_over_all_random_words(y):
    u = np.arange(65536, dtype=np.int64)
    yy = np.full(65536, y, dtype=np.float32)
    codes = o.e2m1_encode_sr(yy, u)
    a = min(abs(float(np.float32(y))), 6.0)
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    lo = max(i for i, m in enumerate(mags) if m <= a)
    hi = min(lo + 1, 7)
    ups = int(np.sum(codes == hi)) if hi != lo else 0
    frac = 0.0 if hi == lo else (a - mags[lo]) / (mags[hi] - mags[lo])
    assert ups == math.floor(frac * 65536)
    # the words that round up are the largest ones (u16 >= 2^16 (1 - frac))
    if ups:
        assert np.all(codes[65536 - ups:] == hi) and np.all(codes[:65536 - ups] == lo)
    assert np.all((codes == lo) | (codes == hi))
    # negative inputs mirror
    assert np.array_equal(o.e2m1_encode_sr(-yy, u), codes | 8)


def test_sr_grid_values_never_move():
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    y = np.repeat(mags, 65536)
    u = np.tile(np.arange(65536), 8)
    assert np.array_equal(o.e2m1_encode_sr(y, u), np.repeat(np.arange(8), 65536))


def test_sr_is_unbiased():
    # Resumen tecnico §2: stochastic rounding removes the systematic bias of
    # deterministic rounding. Mean of N draws vs x, per element.
    rng = np.random.default_rng(5)
    x = rng.laplace(0, 1e-3, (16, 256)).astype(np.float32)
    n = 256
    acc = np.zeros(x.shape, dtype=np.float64)
    acc2 = np.zeros(x.shape, dtype=np.float64)
    for off in range(n):
        q = o.quantize(x, rounding="sr", seed=7, offset=off, outputs=("row",))["row"]
        d = o.dequantize(q.codes, q.scales, q.tensor_scale).astype(np.float64)
        acc += d
        acc2 += d * d
    mean = acc / n
    q0 = o.quantize(x, outputs=("row",))["row"]
    sf = np.repeat(o.e4m3_decode(q0.scales), 16, axis=1) * float(q0.tensor_scale)
    y = np.abs(x.astype(np.float64)) / sf
    sat = y >= 6.0
    # step of the E2M1 interval that contains |y|
    step = np.select([y < 2, y < 4], [0.5, 1.0], 2.0) * sf
    p = np.clip((np.abs(x) - np.floor(np.abs(x) / step) * step) / step, 0, 1)
    sigma = step * np.sqrt(p * (1 - p))
    bound = 5 * sigma / math.sqrt(n) + step * 2.0 ** -16 + 1e-12
    ok = np.abs(mean - x) <= bound
    assert np.all(ok | sat), float(np.max(np.abs(mean - x)[~sat] / bound[~sat]))
    # round to nearest is biased on the same data (sanity of the comparison)
    d_rn = o.dequantize(q0.codes, q0.scales, q0.tensor_scale).astype(np.float64)
    assert np.abs(np.mean(d_rn - x)) >= 0 and np.mean(np.abs(mean - x)) < np.mean(np.abs(d_rn - x))


def test_memory_bits_per_element():
    # deultimominuto.info / news.hamidun.com: about half the memory of FP8.
    r, c = 8192, 5120
    q_bytes = r * c // 2 + r * c // 16 + 4
    bits = 8 * q_bytes / (r * c)
    assert abs(bits - 4.5) < 1e-6
    assert abs(8 / bits - 1.777) < 1e-3


def test_rht_quantize_uses_post_transform_amax():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    q = o.rht_quantize(x, rht_seed=7)
    xt = o.rht(x, 7)
    assert q.amax == np.float32(np.max(np.abs(xt)))
    assert q.codes.shape == (32, 32) and q.scales.shape == (32, 4)
    ref = o.quantize(xt, outputs=("col",))["col"]
    assert np.array_equal(ref.codes, q.codes) and np.array_equal(ref.scales, q.scales)
