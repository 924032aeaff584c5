"""Pins of the feedforward oracle (oracle/ffn.py) against what the mathematics fixes.

- silu at known points: silu(0) = 0, silu(1) = 1/(1 + 1/e), silu(z) - silu(-z) = z for every z,
  silu(z) -> z for large z and -> 0 for very negative z.
- A hand-worked example (d_model = 2, d_ff = 1) with every intermediate written out.
- Special cases: W3 = 0 or x = 0 give 0; doubling W2 doubles the output; permuting the hidden
  units (rows of W1 and W3 with the matching columns of W2) changes nothing.
- Rows are independent: the output of a block of rows equals those rows of the whole.
"""
import math

import numpy as np

from oracle.ffn import silu, swiglu_ffn, swiglu_hidden


def test_silu_values():
    assert silu(0.0) == 0.0
    assert abs(silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    z = np.linspace(-7, 7, 29)
    assert np.allclose(silu(z) - silu(-z), z, atol=1e-14)
    assert abs(silu(40.0) - 40.0) < 1e-12 and abs(silu(-40.0)) < 1e-15


def test_handworked_example():
    x = np.array([[1.0, 2.0]])
    w1 = np.array([[0.5, -0.25]])     # x W1^T = 0.5 - 0.5 = 0      -> silu = 0
    w3 = np.array([[1.0, 1.0]])       # x W3^T = 3
    w2 = np.array([[2.0], [-1.0]])
    assert np.array_equal(swiglu_ffn(x, w1, w3, w2), [[0.0, 0.0]])
    w1 = np.array([[1.0, 0.0]])       # x W1^T = 1 -> silu(1) = 1/(1 + e^-1)
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    assert np.allclose(swiglu_hidden(x, w1, w3), [[3.0 * s1]], atol=1e-15)
    assert np.allclose(swiglu_ffn(x, w1, w3, w2), [[6.0 * s1, -3.0 * s1]], atol=1e-14)


def test_special_cases_and_symmetries():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 16))
    w1, w3 = rng.standard_normal((24, 16)), rng.standard_normal((24, 16))
    w2 = rng.standard_normal((16, 24))
    out = swiglu_ffn(x, w1, w3, w2)
    assert np.array_equal(swiglu_ffn(x, w1, np.zeros_like(w3), w2), np.zeros((5, 16)))
    assert np.array_equal(swiglu_ffn(np.zeros_like(x), w1, w3, w2), np.zeros((5, 16)))
    assert np.allclose(swiglu_ffn(x, w1, w3, 2 * w2), 2 * out, atol=1e-12)
    perm = rng.permutation(24)
    assert np.allclose(swiglu_ffn(x, w1[perm], w3[perm], w2[:, perm]), out, atol=1e-12)


def test_rows_are_independent():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((12, 8))
    w1, w3, w2 = rng.standard_normal((10, 8)), rng.standard_normal((10, 8)), rng.standard_normal((8, 10))
    out = swiglu_ffn(x, w1, w3, w2)
    for r0, r1 in ((0, 5), (5, 12), (3, 4)):
        assert np.allclose(swiglu_ffn(x[r0:r1], w1, w3, w2), out[r0:r1], atol=1e-13)
