"""Pins of the oracle's NVFP4 GEMM reference.

* A pure-Python triple loop over decoded codes and scale bytes on a tiny case
  (brute force; it shares only the codec tables, which are pinned elsewhere).
* Closed form: every code 0x2 (1.0) with scale 0x38 (1.0) and S = 1 gives
  C = K in every entry.
* B with one unit row per output column selects the dequantized A columns.
* Operands with 16x16 scale grids (weights) agree with the same operand
  expressed with 1x16 row scales.
"""

import numpy as np

import oracle as o


def _rand_q(rows, cols, seed):
    rng = np.random.default_rng(seed)
    return o.quantize(rng.standard_normal((rows, cols)).astype(np.float32), outputs=("row",))["row"]


def test_triple_loop_tiny():
    a = _rand_q(4, 32, 0)
    b = _rand_q(3, 32, 1)
    c = o.gemm(a.codes, a.scales, a.tensor_scale, "1d", b.codes, b.scales, b.tensor_scale, "1d")
    ca, cb = o.unpack_codes(a.codes), o.unpack_codes(b.codes)
    for m in range(4):
        for n in range(3):
            acc = 0.0
            for k in range(32):
                va = float(o.e2m1_decode(ca[m, k])) * float(o.e4m3_decode(a.scales[m, k // 16]))
                vb = float(o.e2m1_decode(cb[n, k])) * float(o.e4m3_decode(b.scales[n, k // 16]))
                acc += float(np.float32(np.float32(va) * a.tensor_scale)) * float(
                    np.float32(np.float32(vb) * b.tensor_scale))
            assert abs(c[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_all_ones_closed_form():
    m, n, k = 32, 48, 160
    a_codes = np.full((m, k // 2), 0x22, dtype=np.uint8)
    a_sc = np.full((m, k // 16), 0x38, dtype=np.uint8)
    b_codes = np.full((n, k // 2), 0x22, dtype=np.uint8)
    b_sc = np.full((n // 16, k // 16), 0x38, dtype=np.uint8)
    c = o.gemm(a_codes, a_sc, np.float32(1), "1d", b_codes, b_sc, np.float32(1), "2d")
    assert np.array_equal(c, np.full((m, n), float(k)))


def test_unit_rows_select_columns():
    a = _rand_q(16, 64, 2)
    k = 64
    cols = [0, 5, 17, 63]
    b_codes = np.zeros((len(cols), k), dtype=np.uint8)
    for i, col in enumerate(cols):
        b_codes[i, col] = 0x2  # 1.0
    b_sc = np.full((len(cols), k // 16), 0x38, dtype=np.uint8)
    c = o.gemm(a.codes, a.scales, a.tensor_scale, "1d", o.pack_codes(b_codes), b_sc, np.float32(1), "1d")
    deq = o.dequantize(a.codes, a.scales, a.tensor_scale)
    assert np.array_equal(c, deq[:, cols].astype(np.float64))


def test_2d_grid_equals_expanded_row_scales():
    w = (0.02 * np.random.default_rng(3).standard_normal((32, 64))).astype(np.float32)
    q = o.quantize_2d(w)["row"]
    a = _rand_q(16, 64, 4)
    c2d = o.gemm(a.codes, a.scales, a.tensor_scale, "1d", q.codes, q.scales, q.tensor_scale, "2d")
    rows = np.repeat(q.scales, 16, axis=0)
    c1d = o.gemm(a.codes, a.scales, a.tensor_scale, "1d", q.codes, rows, q.tensor_scale, "1d")
    assert np.array_equal(c2d, c1d)
