"""Pins for the oracle's Hadamard rotation (CPU only): the float64 transform
against scipy's Sylvester matrix, the float32 kernel-order transform against
the float64 one within its rounding bound, self-inverse and dot products."""

import numpy as np
import pytest
import scipy.linalg

from oracle import rotate


@pytest.mark.parametrize("d", [2, 8, 64, 128])
def test_f64_transform_is_the_normalised_sylvester_matrix(d):
    h = scipy.linalg.hadamard(d).astype(np.float64) / np.sqrt(d)
    eye = np.eye(d)
    # Row i of the output for input e_j is H[j, i]; H is symmetric.
    np.testing.assert_allclose(rotate.hadamard_f64(eye, axis=1), h, atol=1e-15)
    x = np.random.default_rng(d).standard_normal((7, d))
    np.testing.assert_allclose(rotate.hadamard_f64(x, axis=1), x @ h.T, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
def test_f32_kernel_order_within_rounding_of_f64(d):
    """Stage s (s = 1..log2 D) rounds values of magnitude at most 2^s max|x|,
    each by at most 2^-24 of that, so before the scaling the error is below
    2^-24 * 2D * max|x|; after the 1/sqrt(D) multiply (one more rounding of
    a value at most sqrt(D) max|x|) it is below 3 sqrt(D) 2^-24 max|x|.  A
    wrong pairing or sign gives errors of order max|x| instead."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((50, d)) * np.exp(rng.uniform(-5, 5, (50, 1)))).astype(np.float32)
    x[::5, 3] *= 50
    got = rotate.hadamard_f32(x, axis=1).astype(np.float64)
    ref = rotate.hadamard_f64(x.astype(np.float64), axis=1)
    bound = 3 * np.sqrt(d) * 2.0 ** -24 * np.abs(x.astype(np.float64)).max(axis=1, keepdims=True)
    assert (np.abs(got - ref) <= bound).all()
    assert got.dtype == np.float64 and rotate.hadamard_f32(x).dtype == np.float32


def test_self_inverse_and_dot_products():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((16, 128))
    k = rng.standard_normal((300, 128))
    k[:, 5] *= 30                                    # an outlier channel
    np.testing.assert_allclose(rotate.hadamard_f64(rotate.hadamard_f64(q)), q, atol=1e-13)
    np.testing.assert_allclose(rotate.hadamard_f64(q) @ rotate.hadamard_f64(k).T, q @ k.T, rtol=1e-12, atol=1e-10)
    # The rotation spreads the outlier channel: the rotated rows' largest
    # entry is far below the original's.
    assert np.abs(rotate.hadamard_f64(k)).max() < 0.5 * np.abs(k).max()
