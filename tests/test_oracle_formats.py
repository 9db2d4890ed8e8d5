"""Pins of the oracle's E2M1 and E4M3 codecs against things other than itself.

* E2M1 values: the closed form of a 1-sign / 2-exponent (bias 1) /
  1-mantissa-bit float, written out as a literal table here.
* E2M1 round-to-nearest-even: an independent route -- round the significand
  to one bit with numpy's rint (ties to even) in each binade -- over every
  float32 near every tie and grid point, plus random values.
* E4M3 (FN): literal byte values, and torch's float8_e4m3fn CPU cast (round to
  nearest even) for every non-negative float32 near every E4M3 midpoint below
  464; saturation by hand above.
"""

import numpy as np
import pytest
import torch

import oracle as o

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_all_16_codes():
    got = o.e2m1_decode(np.arange(16))
    want = E2M1_TABLE + [-v for v in E2M1_TABLE]
    assert np.array_equal(got[:8], np.array(want[:8]))
    assert np.array_equal(got[8:], np.array(want[8:]))
    assert np.all(np.signbit(got[8:]))  # code 8 is -0
    # 16 codes, 15 distinct numbers (+0 and -0 compare equal)
    assert len(set(got.tolist())) == 15


def _rn_by_significand(y: np.ndarray) -> np.ndarray:
    """E2M1 RN via rounding the significand to 1 bit with np.rint per binade."""
    a = np.abs(y.astype(np.float64))
    out = np.empty_like(a)
    small = a < 1.0
    out[small] = np.rint(a[small] * 2.0) / 2.0  # spacing 0.5 below 1
    big = ~small
    _, e = np.frexp(a[big])  # a = f * 2^e, f in [0.5, 1)
    spacing = np.ldexp(1.0, e - 2)  # binade [2^(e-1), 2^e) has spacing 2^(e-2)
    out[big] = np.rint(a[big] / spacing) * spacing
    out = np.minimum(out, 6.0)
    lut = {v: i for i, v in enumerate(E2M1_TABLE)}
    mag = np.array([lut[v] for v in out.tolist()], dtype=np.uint8)
    return mag | (np.signbit(y).astype(np.uint8) << 3)


def _neighbourhood(points, n):
    """All float32 within n ulps of each point."""
    pts = np.asarray(points, dtype=np.float32).view(np.int32)
    k = np.arange(-n, n + 1, dtype=np.int32)
    vals = (pts[:, None] + k[None, :]).reshape(-1)
    vals = vals[vals >= 0].view(np.float32)
    return vals


def test_e2m1_rn_matches_significand_rounding():
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    grid = E2M1_TABLE[1:] + [7.0, 8.0, 12.0]
    y = _neighbourhood(ties + grid, 4096)
    rng = np.random.default_rng(123)
    rand = (rng.standard_normal(200_000) * np.exp2(rng.integers(-12, 6, 200_000))).astype(np.float32)
    special = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-38, 3.4e38, -3.4e38, 6.0, -6.0], dtype=np.float32)
    y = np.concatenate([y, -y, rand, special])
    assert np.array_equal(o.e2m1_encode_rn(y), _rn_by_significand(y))


def test_e2m1_rn_ties_go_to_even_code():
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    assert o.e2m1_encode_rn(ties).tolist() == [0, 2, 2, 4, 4, 6, 6]
    up = np.nextafter(ties, np.float32(np.inf))
    down = np.nextafter(ties, np.float32(0))
    assert o.e2m1_encode_rn(up).tolist() == [1, 2, 3, 4, 5, 6, 7]
    assert o.e2m1_encode_rn(down).tolist() == [0, 1, 2, 3, 4, 5, 6]


def test_e2m1_rn_sign_symmetry_and_negative_zero():
    y = np.linspace(0, 10, 10001, dtype=np.float32)
    assert np.array_equal(o.e2m1_encode_rn(-y), o.e2m1_encode_rn(y) | 8)
    assert o.e2m1_encode_rn(np.float32(-0.1)) == 8
    assert o.e2m1_encode_rn(np.float32(0.0)) == 0


def test_e2m1_rn_round_trip():
    codes = np.arange(16)
    assert np.array_equal(o.e2m1_encode_rn(o.e2m1_decode(codes).astype(np.float32)), codes)


def test_e2m1_rn_rejects_non_finite():
    with pytest.raises(ValueError):
        o.e2m1_encode_rn(np.array([np.nan], dtype=np.float32))


# ---------------------------------------------------------------- E4M3


def test_e4m3_decode_literal_bytes():
    d = o.e4m3_decode
    assert d(0x00) == 0.0
    assert d(0x01) == 2.0 ** -9
    assert d(0x07) == 7 * 2.0 ** -9
    assert d(0x08) == 2.0 ** -6
    assert d(0x38) == 1.0
    assert d(0x23) == 0.171875
    assert d(0x30) == 0.5
    assert d(0x7E) == 448.0
    assert d(0x7D) == 416.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0xB8) == -1.0
    assert np.signbit(d(0x80)) and d(0x80) == 0.0
    vals = o.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)  # strictly increasing 0x00..0x7E
    assert np.array_equal(o.e4m3_decode(np.arange(0x80, 0xFF)), -vals)


def _torch_e4m3(t: np.ndarray) -> np.ndarray:
    return torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_cast_below_464():
    vals = o.e4m3_decode(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, [464.0]])
    t = _neighbourhood(pts, 2048)
    rng = np.random.default_rng(7)
    rand = (rng.random(300_000) * np.exp2(rng.integers(-16, 9, 300_000))).astype(np.float32)
    t = np.concatenate([t, rand])
    t = t[(t >= 0) & (t < 464.0)]
    assert np.array_equal(o.e4m3_encode(t), _torch_e4m3(t))


def test_e4m3_encode_saturates():
    t = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1e30, 3.4e38], dtype=np.float32)
    assert o.e4m3_encode(t).tolist() == [0x7E] * len(t)


def test_e4m3_encode_tiny_values():
    t = np.array([0.0, 2.0 ** -11, 2.0 ** -10, np.nextafter(np.float32(2.0 ** -10), np.float32(1)),
                  2.0 ** -9, 1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9], dtype=np.float32)
    # 2^-10 is the midpoint between 0 and 2^-9: ties to even -> 0
    assert o.e4m3_encode(t).tolist() == [0, 0, 0, 1, 1, 2, 2]


def test_e4m3_encode_rejects_negative_or_nan():
    with pytest.raises(ValueError):
        o.e4m3_encode(np.array([-1.0], dtype=np.float32))
    with pytest.raises(ValueError):
        o.e4m3_encode(np.array([np.nan], dtype=np.float32))
