"""The parity checker itself: a comparison must fail on any element where the two sides
disagree, non-finite values included, and pass only where both agree."""
import numpy as np
import pytest

from harness import assert_close, close_mask


def test_equal_and_within_tolerance_pass():
    ref = np.array([[1.0, -2.0, 0.0, 1e3]])
    assert assert_close(ref + 0.01, ref, 2e-2, 1e-2, "ok") <= 0.0100001
    assert assert_close(ref.copy(), ref, 0.0, 0.0, "exact") == 0.0


def test_outside_tolerance_fails():
    ref = np.ones((2, 3))
    g = ref.copy()
    g[1, 2] = 1.04
    with pytest.raises(AssertionError):
        assert_close(g, ref, 2e-2, 1e-2, "one off")


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite_on_one_side_fails(bad):
    ref = np.ones((1, 3))
    g = ref.copy()
    g[0, 1] = bad
    with pytest.raises(AssertionError):
        assert_close(g, ref, 2e-2, 1e-2, "gpu non-finite")
    with pytest.raises(AssertionError):
        assert_close(ref, g, 2e-2, 1e-2, "oracle non-finite")


def test_finite_against_infinity_fails():
    # a relative tolerance makes the limit infinite; that must not admit a finite value
    ref = np.array([np.inf, -np.inf])
    with pytest.raises(AssertionError):
        assert_close(np.array([1e30, -1e30]), ref, 2e-2, 1e-2, "finite vs inf")


def test_same_nonfinite_on_both_sides_passes():
    ref = np.array([np.nan, np.inf, -np.inf, 1.0])
    g = np.array([np.nan, np.inf, -np.inf, 1.0])
    assert_close(g, ref, 0.0, 0.0, "both")
    assert close_mask(g, ref, 0.0, 0.0).all()


def test_opposite_infinities_fail():
    with pytest.raises(AssertionError):
        assert_close(np.array([np.inf]), np.array([-np.inf]), 2e-2, 1e-2, "inf vs -inf")


def test_shape_mismatch_fails():
    with pytest.raises(AssertionError):
        assert_close(np.ones((2, 2)), np.ones((2, 3))[:, :2].T.reshape(2, 2)[:1], 0.1, 0.1, "shape")
