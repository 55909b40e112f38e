"""Pins for oracle.rope: invariants of a rotation and values fixed by the
reading (interleaved pairs, theta_j = base^(-2j/d))."""
import math

import numpy as np
import pytest

from oracle.rope import rope, rope_angles


def test_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((5, 64))
    assert np.array_equal(rope(x, 0, 10000.0), x)


def test_norm_preserved_per_pair():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 64))
    y = rope(x, rng.integers(0, 200000, 7), 10000.0)
    nx = x[:, 0::2] ** 2 + x[:, 1::2] ** 2
    ny = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    assert np.allclose(nx, ny, rtol=1e-13, atol=0)


def test_relative_position_property():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in [(0, 5), (17, 17), (1000, 3), (131071, 65536)]:
        lhs = rope(q, m, 10000.0) @ rope(k, n, 10000.0)
        rhs = q @ rope(k, n - m, 10000.0)
        # fp64 angles p*theta carry an absolute error of about p * 2^-52
        tol = 4e-16 * (m + n + 1) * np.linalg.norm(q) * np.linalg.norm(k)
        assert abs(lhs - rhs) <= tol


def test_two_dims_rotate_by_p_radians_counterclockwise():
    # d = 2: theta_0 = 1, so position p rotates by p radians
    for p in [1, 2, 7, 100]:
        y = rope(np.array([1.0, 0.0]), p, 10000.0)
        assert np.allclose(y, [math.cos(p), math.sin(p)], rtol=0, atol=1e-15)
        y = rope(np.array([0.0, 1.0]), p, 10000.0)
        assert np.allclose(y, [-math.sin(p), math.cos(p)], rtol=0, atol=1e-15)


def test_pair_frequencies():
    # d = 4, base 10000: pair 0 at theta 1, pair 1 at theta 10000^(-1/2) = 0.01
    y = rope(np.array([1.0, 0.0, 1.0, 0.0]), 3, 10000.0)
    assert np.allclose(y, [math.cos(3), math.sin(3), math.cos(0.03), math.sin(0.03)], atol=1e-15)
    ang = rope_angles(np.array([1]), 64, 10000.0)[0]
    assert ang[0] == 1.0 and ang[31] == pytest.approx(10000.0 ** (-62 / 64), rel=1e-15)
    assert np.all(np.diff(ang) < 0)


def test_inverse_rotation():
    x = np.random.default_rng(4).standard_normal(64)
    assert np.allclose(rope(rope(x, 4095, 10000.0), -4095, 10000.0), x, atol=1e-12)


def test_odd_width_rejected():
    with pytest.raises(ValueError):
        rope(np.zeros(3), 1, 10000.0)
