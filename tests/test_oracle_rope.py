"""Pins for oracle.rope: complex-multiplication form, inverse, relative-position invariance, YaRN segments."""
import math

import numpy as np
import pytest

from oracle import rope


def test_plain_frequencies():
    f = rope.inv_freq(64, 10000.0)
    assert f.shape == (32,)
    assert f[0] == 1.0
    assert math.isclose(f[1], 10000.0 ** (-2.0 / 64), rel_tol=1e-15)
    assert np.all(np.diff(f) < 0)


def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 64))
    f = rope.inv_freq(16, 10000.0)
    pos = 1234567
    y = rope.rotate_tail(x, pos, f)
    z = x[:, 48::2] + 1j * x[:, 49::2]
    z = z * np.exp(1j * pos * f)
    assert np.allclose(y[:, 48::2], z.real, atol=1e-12) and np.allclose(y[:, 49::2], z.imag, atol=1e-12)
    assert np.array_equal(y[:, :48], x[:, :48])


def test_inverse_undoes_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 512))
    f = rope.inv_freq(64, 160000.0, 16.0, 65536)
    for pos in [0, 1, 65535, 1048575]:
        y = rope.rotate_tail(rope.rotate_tail(x, pos, f), pos, f, inverse=True)
        assert np.allclose(y, x, atol=1e-12)


def test_score_depends_on_relative_position_only():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(512), rng.standard_normal(512)
    f = rope.inv_freq(64, 160000.0, 16.0, 65536)
    a = rope.rotate_tail(q, 5000, f) @ rope.rotate_tail(k, 4000, f)
    b = rope.rotate_tail(q, 905000, f) @ rope.rotate_tail(k, 904000, f)
    assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)


def test_yarn_factor_one_is_plain():
    assert np.array_equal(rope.inv_freq(64, 160000.0, 1.0, 65536), rope.inv_freq(64, 160000.0))


def test_yarn_segments():
    base = rope.inv_freq(64, 160000.0)
    y = rope.inv_freq(64, 160000.0, 16.0, 65536)
    turns = 65536 / (2 * math.pi / base)
    hi = turns > 32
    lo = turns < 1
    assert hi.any() and lo.any()
    assert np.allclose(y[hi], base[hi], rtol=0, atol=0)
    assert np.allclose(y[lo], base[lo] / 16.0, rtol=1e-15)
    mid = ~hi & ~lo
    assert np.all((y[mid] < base[mid]) & (y[mid] > base[mid] / 16.0))
