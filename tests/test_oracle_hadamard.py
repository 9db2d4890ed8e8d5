"""Pins of the oracle's 16-point random Hadamard transform.

* The matrix equals scipy.linalg.hadamard(16) (Sylvester construction,
  natural order) -- a library routine, not the popcount formula the oracle
  uses.
* H H^T = 16 I exactly; the transform keeps the 2-norm of every 16-block;
  (1/4) D H^T undoes it; a single spike a*e_k maps to (a d_k / 4) H[:, k].
* Applying the transform to both weight-gradient operands leaves dY^T X
  unchanged (it is orthonormal and the same d is used on both).
"""

import numpy as np
import scipy.linalg

import oracle as o


def test_matrix_is_sylvester_hadamard():
    assert np.array_equal(o.hadamard16(), scipy.linalg.hadamard(16))


def test_orthogonality():
    h = o.hadamard16()
    assert np.array_equal(h @ h.T, 16 * np.eye(16, dtype=np.int64))


def test_signs_are_fixed_plus_minus_one():
    d = o.rht_signs(7)
    assert d.shape == (16,) and set(np.unique(d).tolist()) <= {-1, 1}
    assert np.array_equal(d, o.rht_signs(7))
    assert not np.array_equal(o.rht_signs(7), o.rht_signs(8)) or not np.array_equal(
        o.rht_signs(7), o.rht_signs(9))


def test_norm_preserved_and_inverse():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 24)).astype(np.float32)
    y = o.rht(x, 7).astype(np.float64)
    xb = x.astype(np.float64).reshape(4, 16, 24)
    yb = y.reshape(4, 16, 24)
    assert np.allclose(np.linalg.norm(xb, axis=1), np.linalg.norm(yb, axis=1), rtol=1e-6)
    h = scipy.linalg.hadamard(16).astype(np.float64)
    d = o.rht_signs(7).astype(np.float64)
    back = np.einsum("i,ji,bjc->bic", d, h, yb) / 4.0  # (1/4) D H^T y
    assert np.allclose(back, xb, rtol=0, atol=1e-6)


def test_single_spike():
    d = o.rht_signs(11)
    h = scipy.linalg.hadamard(16)
    for k in (0, 5, 15):
        x = np.zeros((16, 1), dtype=np.float32)
        x[k, 0] = 8.0
        y = o.rht(x, 11)[:, 0]
        assert np.array_equal(y, (8.0 * d[k] / 4.0) * h[:, k].astype(np.float32))


def test_wgrad_product_invariant():
    rng = np.random.default_rng(1)
    dy = rng.laplace(0, 1e-3, (128, 40)).astype(np.float32)
    x = rng.standard_normal((128, 24)).astype(np.float32)
    ref = dy.astype(np.float64).T @ x.astype(np.float64)
    got = o.rht(dy, 7).astype(np.float64).T @ o.rht(x, 7).astype(np.float64)
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-9)


def test_outliers_spread():
    # Lo esencial item 3 / Resumen tecnico RHT: the transform spreads an outlier
    # over its 16-block, so the block's max shrinks relative to its norm.
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1024, 8)).astype(np.float32)
    x[::97, :] *= 50
    y = o.rht(x, 7)
    kurt = lambda v: float(np.mean((v - v.mean()) ** 4) / np.var(v) ** 2)
    assert kurt(y) < kurt(x) / 2
