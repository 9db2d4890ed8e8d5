"""Pins of the MXFP4 oracle (the pages' comparison format).

* E8M0 bytes against float32 exponent fields: byte b >= 1 is the float32
  with exponent field b and a zero mantissa; byte 0 is the float32 subnormal
  2^-127; 255 is NaN.
* The scale choice puts every block amax in [4, 8) after scaling, and no
  other byte does; brute force over a range of amax values.
* A hand-worked block.
* Power-of-two invariance: scaling a row by 2^k keeps every code and adds k
  to every scale byte.
* The GEMM against a triple loop on a tiny shape.
* NVFP4 (16-element blocks, E4M3 scales) quantizes Gaussian data with a
  smaller error than MXFP4 (the pages' comparison, Resumen técnico §2).
"""

import numpy as np
import pytest

import oracle as o


def test_e8m0_bytes_are_float32_exponent_fields():
    for b in range(1, 255):
        f = np.array([b << 23], dtype=np.uint32).view(np.float32)[0]
        assert o.e8m0_decode(b) == float(f), b
    sub = np.array([1 << 22], dtype=np.uint32).view(np.float32)[0]  # 2^-127
    assert o.e8m0_decode(0) == float(sub)
    assert np.isnan(o.e8m0_decode(255))


def test_scale_choice_maps_amax_into_4_8():
    rng = np.random.default_rng(0)
    amax = np.concatenate([
        np.float32(2.0) ** rng.integers(-120, 120, 4000).astype(np.float32)
        * rng.uniform(1.0, 2.0, 4000).astype(np.float32),
        np.array([1.0, 2.0, 4.0, 7.999, 8.0, 0.75, 3e-30], np.float32)])
    b = o.mx_scale_bytes(amax)
    y = amax.astype(np.float64) / o.e8m0_decode(b)
    assert np.all((y >= 4.0) & (y < 8.0))
    # brute force: the only byte with that property
    for a, bb in zip(amax[:200], b[:200]):
        ok = [k for k in range(255) if 4.0 <= float(a) / float(o.e8m0_decode(k)) < 8.0]
        assert ok == [int(bb)]
    assert o.mx_scale_bytes(np.float32(0.0)) == 0


def test_hand_worked_block():
    # Block max 3.0: floor(log2 3) = 1, so b = 1 - 2 + 127 = 126 and the
    # scale is 2^-1; elements are doubled before rounding to E2M1.
    x = np.zeros((1, 32), np.float32)
    x[0, :8] = [3.0, -0.3, 1.3, 0.1, 0.125, -2.6, 0.75, 1.75]
    # doubled: 6 -> 6 (code 7); -0.6 -> -0.5 (0x9); 2.6 -> 3 (code 5);
    # 0.2 -> 0 (code 0); 0.25 -> tie between 0 and 0.5, even code 0;
    # -5.2 -> -6, nearer than -4 (0xF); 1.5 -> 1.5 (code 3); 3.5 -> tie
    # between 3 and 4 -> 4 (code 6)
    codes, scales = o.mx_quantize(x)
    assert scales.tolist() == [[126]]
    want = [7, 9, 5, 0, 0, 15, 3, 6] + [0] * 24
    assert o.unpack_codes(codes)[0].tolist() == want
    d = o.mx_dequantize(codes, scales)
    assert d[0, :8].tolist() == [3.0, -0.25, 1.5, 0.0, 0.0, -3.0, 0.75, 2.0]


def test_clipping_of_power_of_two_scales():
    # amax 7.5 * 2^-3: scaled to 7.5, which saturates to 6
    x = np.full((1, 32), 0.01, np.float32)
    x[0, 5] = 7.5 / 8
    codes, scales = o.mx_quantize(x)
    assert o.unpack_codes(codes)[0, 5] == 7
    assert o.mx_dequantize(codes, scales)[0, 5] == 6.0 / 8


@pytest.mark.parametrize("k", [-20, -3, 1, 17])
def test_power_of_two_invariance(k):
    rng = np.random.default_rng(3)
    x = rng.normal(size=(8, 128)).astype(np.float32)
    c0, s0 = o.mx_quantize(x)
    c1, s1 = o.mx_quantize((x * np.float32(2.0) ** k).astype(np.float32))
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1.astype(np.int64), s0.astype(np.int64) + k)


def test_gemm_triple_loop():
    rng = np.random.default_rng(4)
    a = rng.normal(size=(3, 64)).astype(np.float32)
    b = rng.normal(size=(5, 64)).astype(np.float32)
    qa, sa = o.mx_quantize(a)
    qb, sb = o.mx_quantize(b)
    got = o.mx_gemm(qa, sa, qb, sb)
    ua, ub = o.unpack_codes(qa), o.unpack_codes(qb)
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    val = lambda c: (-1 if c & 8 else 1) * mags[c & 7]
    for m in range(3):
        for n in range(5):
            acc = 0.0
            for kk in range(64):
                acc += (val(int(ua[m, kk])) * 2.0 ** (int(sa[m, kk // 32]) - 127)
                        * val(int(ub[n, kk])) * 2.0 ** (int(sb[n, kk // 32]) - 127))
            assert got[m, n] == acc


def test_nvfp4_quantizes_more_accurately_than_mxfp4():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(64, 512)).astype(np.float32)
    qm, sm = o.mx_quantize(x)
    err_mx = np.mean((o.mx_dequantize(qm, sm) - x) ** 2)
    q = o.quantize(x, outputs=("row",))["row"]
    err_nv = np.mean((o.dequantize(q.codes, q.scales, q.tensor_scale) - x) ** 2)
    assert err_nv < err_mx
