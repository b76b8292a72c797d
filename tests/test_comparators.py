"""CPU checks of the parity comparators the GPU tests use."""

import numpy as np
import pytest

from tests.gpu_util import assert_bits_equal, assert_f32_bits_equal_nan_as_nan


def test_nan_matches_any_nan_only():
    assert_f32_bits_equal_nan_as_nan(np.uint32([0x7FC10000, 1, 0x7F800000]),
                                     np.uint32([0xFFC00000, 1, 0x7F800000]), "nan payloads")
    with pytest.raises(AssertionError):                      # NaN against infinity
        assert_f32_bits_equal_nan_as_nan(np.uint32([0x7FC00000]), np.uint32([0x7F800000]), "nan vs inf")
    with pytest.raises(AssertionError):                      # any other bit differs
        assert_f32_bits_equal_nan_as_nan(np.uint32([0x3F800000]), np.uint32([0x3F800001]), "one ulp")
    with pytest.raises(AssertionError):                      # signed zeros differ
        assert_f32_bits_equal_nan_as_nan(np.uint32([0x80000000]), np.uint32([0]), "zeros")


def test_bits_equal_is_exact():
    assert_bits_equal(np.uint32([1, 2]), np.uint32([1, 2]), "same")
    with pytest.raises(AssertionError):
        assert_bits_equal(np.uint32([0x7FC10000]), np.uint32([0x7FC00000]), "nan payload")
