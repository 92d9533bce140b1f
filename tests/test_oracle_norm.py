"""Pins of the RMSNorm oracle (oracle.norm): closed forms, invariances and an
independent float64 loop."""
import math

import numpy as np
import pytest

from oracle import norm, quant


def test_constant_rows_closed_form():
    # a row of c's has mean square c^2: y = c * g / sqrt(c^2 + eps)
    x = np.array([[3.0] * 16, [-0.5] * 16, [0.0] * 16])
    g = np.linspace(0.5, 2.0, 16)
    y = norm.rmsnorm(x, g, 1e-6)
    for r, c in enumerate([3.0, -0.5, 0.0]):
        np.testing.assert_allclose(y[r], c * g / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)


def test_matches_scalar_loop():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 48)).astype(np.float32)
    g = rng.standard_normal(48).astype(np.float32)
    y = norm.rmsnorm(x, g, 1e-5)
    for r in range(5):
        ss = 0.0
        for c in range(48):
            ss += float(x[r, c]) ** 2
        inv = 1.0 / math.sqrt(ss / 48 + 1e-5)
        for c in range(48):
            assert abs(y[r, c] - float(x[r, c]) * inv * float(g[c])) <= 1e-12 * max(1.0, abs(y[r, c]))


def test_unit_gain_rows_have_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 64)) * 5.0
    y = norm.rmsnorm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(norm.rmsnorm(x * 1024.0, np.ones(64), 0.0), y, rtol=1e-13)   # with eps = 0


def test_quantize_is_quantisation_of_rounded_norm():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 32)).astype(np.float32)
    g = (1.0 + 0.1 * rng.standard_normal(32)).astype(np.float32)
    q = norm.rmsnorm_quantize(x, g, 1e-6)
    ref = quant.quantize(norm.rmsnorm(x, g, 1e-6).astype(np.float32))
    assert np.array_equal(q.codes, ref.codes) and np.array_equal(q.scales, ref.scales) and q.gs == ref.gs
    # the normalised block maximum maps to +-6 in every block (the quantiser's invariant)
    dec = quant.dequantize(q)
    y = norm.rmsnorm(x, g, 1e-6)
    blk = np.abs(y).reshape(4, 2, 16).max(-1)
    assert np.all(np.abs(dec).reshape(4, 2, 16).max(-1) <= blk * 1.1 + 1e-12)


def test_zero_row_gives_zero_codes():
    q = norm.rmsnorm_quantize(np.zeros((2, 32), np.float32), np.ones(32, np.float32), 1e-6)
    assert not np.any(q.scales)
    assert pytest.approx(float(q.gs)) == float(np.float32(np.float32(1e-8) / np.float32(2688.0)))
