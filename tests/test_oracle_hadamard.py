"""Pins of the oracle's Hadamard rotation: orthogonality, the explicit +-1
matrix on inputs where fp32 is exact, dot-product invariance, and the fp32
normalisation constant from exact integer arithmetic."""

import numpy as np
import pytest

from oracle import hadamard


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_sylvester_is_hadamard(d):
    h = hadamard.sylvester(d)
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))
    np.testing.assert_array_equal(h, h.T)
    hn = h / np.sqrt(d)
    np.testing.assert_allclose(hn @ hn.T, np.eye(d), atol=1e-14)


@pytest.mark.parametrize("d", [64, 128])
def test_fwht_equals_matrix_on_exact_inputs(d):
    """Small integers keep every butterfly sum exact in fp32, so the transform
    must equal fp32(x @ H) times the fp32 constant, element for element."""
    rng = np.random.default_rng(11)
    x = rng.integers(-50, 50, size=(37, 3, d)).astype(np.float32)
    got = hadamard.fwht_fp32(x)
    exact = (x.astype(np.int64) @ hadamard.sylvester(d)).astype(np.float32)
    np.testing.assert_array_equal(got, exact * hadamard.inv_sqrt_fp32(d))


def test_fwht_butterfly_order_on_one_vector():
    # d = 4: stage h=1 pairs (0,1),(2,3); stage h=2 pairs (0,2),(1,3)
    x = np.array([1.0, 2.0, 3.0, 4.0], np.float32)
    s1 = np.array([3, -1, 7, -1], np.float32)
    s2 = np.array([10, -2, -4, 0], np.float32)
    np.testing.assert_array_equal(hadamard.fwht_fp32(x), s2 * np.float32(0.5))
    assert s1 is not None


def test_rotation_preserves_dot_products():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((20, 128))
    k = rng.standard_normal((30, 128))
    h = hadamard.sylvester(128) / np.sqrt(128)
    np.testing.assert_allclose((q @ h) @ (k @ h).T, q @ k.T, atol=1e-11)
    np.testing.assert_allclose(hadamard.rotate_back_fp64(q @ h), q, atol=1e-12)


def test_inv_sqrt_constants():
    assert hadamard.inv_sqrt_fp32(64) == np.float32(0.125)
    # fp32 nearest to 2**-3.5: c = m * 2**-27 with m a 24-bit integer; check
    # (2m-1)^2 < 2**49 < (2m+1)^2, i.e. |c - 2**-3.5| < half an ulp, exactly.
    c = hadamard.inv_sqrt_fp32(128)
    m = int(np.float64(c) * 2.0 ** 27)
    assert m * 2.0 ** -27 == float(c) and 2 ** 23 <= m < 2 ** 24
    assert (2 * m - 1) ** 2 < 2 ** 49 < (2 * m + 1) ** 2
