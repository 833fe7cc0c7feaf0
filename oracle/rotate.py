"""Hadamard rotation of query and key rows before MXFP4.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "BitDecoding-FP4: Algorithm-System Co-Design for Native FP4 KV Cache
Decoding" (Abstract and the section on key outliers): static smoothing,
Hadamard rotation and scale search suppress key outliers.  An orthonormal
rotation applied to both the query and the key rows leaves every dot
product unchanged while it spreads a few large channels over the block.

Readings taken where the source is silent:
  * The rotation is the normalised Walsh-Hadamard transform of each D-long
    row (D a power of two), H = S_D / sqrt(D) with S_D the Sylvester matrix
    (S_1 = [1], S_2n = [[S_n, S_n], [S_n, -S_n]]).  It is its own inverse.
  * It is applied to the float32 row after the optional Smooth-QK channel
    multiply and before the block quantisation, to Q and K alike (V is not
    rotated).
  * Because it feeds a quantiser, it is defined as the float32 computation
    that the kernel performs: butterflies (a, b) -> (a + b, a - b) on element
    pairs (i, i + h) with i & h = 0, for h = 1, 2, 4, ..., D/2 in that
    order, each result rounded to float32, then one float32 multiply by
    float32(1 / sqrt(D)).  Both sides take every rounding decision the same
    way.

Parity: pinned by tests/test_oracle_rotate.py -- the float64 transform equals
the Sylvester matrix product (scipy.linalg.hadamard), the float32 transform
stays within the rounding bound of that product, applying it twice returns
the row, and dot products are preserved.
"""

import numpy as np


def hadamard_f64(x, axis=-1):
    """The normalised Walsh-Hadamard transform along ``axis`` in float64."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1).copy()
    d = x.shape[-1]
    assert d & (d - 1) == 0, "row length must be a power of two"
    h = 1
    while h < d:
        y = x.reshape(x.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b
        x = y.reshape(x.shape)
        h *= 2
    return np.moveaxis(x / np.sqrt(d), -1, axis)


def hadamard_f32(x, axis=-1):
    """The same transform as the kernel computes it: float32 butterflies in
    stage order h = 1, 2, ..., D/2, then one float32 multiply by
    float32(1/sqrt(D))."""
    x = np.moveaxis(np.asarray(x, dtype=np.float32), axis, -1).copy()
    d = x.shape[-1]
    assert d & (d - 1) == 0, "row length must be a power of two"
    h = 1
    while h < d:
        y = x.reshape(x.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b      # float32 arithmetic
        x = y.reshape(x.shape)
        h *= 2
    x = x * np.float32(1.0 / np.sqrt(float(d)))
    return np.moveaxis(x, -1, axis)
