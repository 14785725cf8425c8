"""The fp32 tolerance rule of tests/parity.py, on hand-made values (CPU)."""

import numpy as np
import pytest

from tests.parity import assert_close_f32


def test_relative_bar_where_nothing_cancels():
    ref = np.array([1.0, -2.0, 3.0])
    mag = np.array([1.0, 2.5, 3.5])  # |ref| >= M / 2: the bar is 1e-5 |ref|
    assert_close_f32(ref * (1 + 0.9e-5), ref, mag)
    with pytest.raises(AssertionError):
        assert_close_f32(ref * (1 + 1.1e-5), ref, mag)


def test_conditioned_bar_only_under_cancellation():
    ref = np.array([1e-3, 0.0])
    mag = np.array([10.0, 4.0])  # |ref| < M / 2: the bar is 1e-5 M
    assert_close_f32(ref + np.array([0.9e-4, -3.9e-5]), ref, mag)
    with pytest.raises(AssertionError):
        assert_close_f32(ref + np.array([1.1e-4, 0.0]), ref, mag)


def test_exact_zero_stays_exact():
    with pytest.raises(AssertionError):
        assert_close_f32(np.array([1e-30]), np.array([0.0]), np.array([0.0]))
