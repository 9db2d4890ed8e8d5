"""Pins of the FP8 (E4M3, per-tensor) oracle, the pages' baseline format.

* Element bytes against an independent implementation: torch's
  float32 -> float8_e4m3fn cast (round to nearest even) for every magnitude
  below 448, signed, over random values and every float32 within a few ulps
  of every E4M3 midpoint; saturation and signed zero by hand.
* Closed forms of the tensor scale (amax 448 -> 1, amax 0 -> 1, powers of
  two, the 2^-100 floor).
* The tensor's largest magnitude always maps to byte 0x7E (448).
* Values that are E4M3 numbers times a power-of-two scale come back exactly.
* Power-of-two invariance of the bytes.
* Round-trip error within half an E4M3 step.
* The column copy is the row copy transposed.
* The GEMM against a pure-Python triple loop, and the all-ones closed form.
"""

import numpy as np
import pytest
import torch

import oracle as o


def torch_e4m3(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_cast_below_448():
    rng = np.random.default_rng(3)
    vals = o.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # all exact in float32
    near = []
    for m in list(mids) + list(vals):
        b = np.float32(m).view(np.uint32)
        near.append((np.arange(-6, 7, dtype=np.int64) + int(b)).astype(np.uint32).view(np.float32))
    near = np.concatenate(near)
    rand = (rng.uniform(-1, 1, 200000) * np.exp2(rng.uniform(-12, 8.8, 200000))).astype(np.float32)
    y = np.concatenate([near, -near, rand])
    y = y[np.abs(y) < 448.0]
    got = o.fp8_encode(y)
    want = torch_e4m3(y)
    # torch keeps the sign of a value that rounds to zero, as F1 does
    assert np.array_equal(got, want)


def test_encode_saturates_and_keeps_zero_sign():
    y = np.array([448.0, 449.0, 464.0, 479.9, 1e30, -500.0, 0.0, -0.0, -1e-30], np.float32)
    got = o.fp8_encode(y)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x80]


def test_tensor_scale_closed_forms():
    assert o.fp8_tensor_scale(448.0) == np.float32(1.0)
    assert o.fp8_tensor_scale(0.0) == np.float32(1.0)
    assert o.fp8_tensor_scale(448.0 * 2.0 ** -90) == np.float32(2.0 ** -90)
    assert o.fp8_tensor_scale(448.0 * 2.0 ** -101) == np.float32(1.0)  # below the floor
    assert o.fp8_tensor_scale(3584.0) == np.float32(8.0)
    assert o.fp8_tensor_scale(1.0) == np.float32(np.float32(1.0) / np.float32(448.0))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_largest_magnitude_maps_to_448(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((64, 96)) * np.exp2(rng.uniform(-20, 20))).astype(np.float32)
    q, _, _ = o.fp8_quantize(x)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q[i] & 0x7F == 0x7E
    assert np.all((q & 0x7F) <= 0x7E)


def test_e4m3_numbers_times_power_of_two_are_exact():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 0x7F, (32, 48)).astype(np.uint8) | (rng.integers(0, 2, (32, 48)).astype(np.uint8) << 7)
    codes[0, 0] = 0x7E  # amax = 448 * 2^j
    for j in (-30, 0, 12):
        x = (o.e4m3_decode(codes) * 2.0 ** j).astype(np.float32)
        q, _, s8 = o.fp8_quantize(x)
        assert s8 == np.float32(2.0 ** j)
        nz = (codes & 0x7F) != 0
        assert np.array_equal(q[nz], codes[nz])
        assert np.array_equal(o.fp8_dequantize(q, s8), x)


def test_power_of_two_invariance():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((40, 64)).astype(np.float32)
    q0, _, s0 = o.fp8_quantize(x)
    for j in (-40, -3, 7, 60):
        q, _, s = o.fp8_quantize((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q, q0)
        assert s == np.float32(s0 * np.float32(2.0 ** j))


def test_round_trip_error_within_half_step():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((128, 64)).astype(np.float32)
    q, _, s8 = o.fp8_quantize(x)
    xh = o.fp8_dequantize(q, s8).astype(np.float64)
    y = np.abs(x.astype(np.float64)) / float(s8)
    normal = y >= 2.0 ** -6
    err = np.abs(xh - x) / float(s8)
    # normal range: half of a 3-bit mantissa step (plus the rounding of x * r)
    assert np.all(err[normal] <= y[normal] * 2.0 ** -4 * (1 + 2.0 ** -20))
    # subnormal range: half of the 2^-9 spacing
    assert np.all(err[~normal] <= 2.0 ** -10 * (1 + 2.0 ** -20))


def test_column_copy_is_the_transpose():
    x = np.random.default_rng(4).standard_normal((48, 80)).astype(np.float32)
    q, qt, _ = o.fp8_quantize(x)
    assert qt.shape == (80, 48) and np.array_equal(qt, q.T)


def test_gemm_triple_loop():
    rng = np.random.default_rng(11)
    m, n, k = 3, 4, 16
    qa = rng.integers(0, 256, (m, k)).astype(np.uint8)
    qb = rng.integers(0, 256, (n, k)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x38
    qb[(qb & 0x7F) == 0x7F] = 0x38
    sa, sb = np.float32(0.375), np.float32(2.0 ** -5)
    got = o.fp8_gemm(qa, sa, qb, sb)
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for t in range(k):
                acc += float(o.e4m3_decode(qa[i, t])) * float(o.e4m3_decode(qb[j, t]))
            assert got[i, j] == np.float32(acc * 0.375 * 2.0 ** -5)


def test_gemm_all_ones():
    qa = np.full((5, 64), 0x38, np.uint8)  # 1.0
    qb = np.full((7, 64), 0x38, np.uint8)
    c = o.fp8_gemm(qa, 0.5, qb, 3.0, out_dtype="bf16")
    assert np.all(c == 96.0)
