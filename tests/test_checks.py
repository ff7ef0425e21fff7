"""The comparison rules of the GPU parity tests must not let a NaN or a wrong infinity pass
(CPU only)."""

import numpy as np
import pytest

from tests import checks


def test_nan_in_gpu_array_fails():
    with pytest.raises(AssertionError):
        checks.assert_close("x", [1.0, np.nan, 2.0], [1.0, 5.0, 2.0], 2e-2)
    assert checks.max_abs([1.0, np.nan, 2.0], [1.0, 5.0, 2.0]) == float("inf")


def test_nan_everywhere_fails():
    with pytest.raises(AssertionError):
        checks.assert_close("x", np.full((3, 4), np.nan), np.zeros((3, 4)), 2e-2)


def test_nan_only_in_reference_fails():
    assert checks.max_abs([1.0, 2.0], [1.0, np.nan]) == float("inf")


def test_equal_infinities_are_equal():
    # an empty row's LSE is -inf on both sides
    assert checks.assert_close("lse", [-np.inf, 0.5], [-np.inf, 0.5 + 1e-4], 1e-3) <= 1e-3


@pytest.mark.parametrize("gpu,ref", [([np.inf], [-np.inf]), ([-np.inf], [0.0]),
                                     ([1.0], [np.inf])])
def test_unequal_infinities_fail(gpu, ref):
    with pytest.raises(AssertionError):
        checks.assert_close("x", gpu, ref, 2e-2)


def test_within_and_beyond_tolerance():
    assert checks.assert_close("x", [1.0, 2.01], [1.0, 2.0], 2e-2) == pytest.approx(0.01)
    with pytest.raises(AssertionError):
        checks.assert_close("x", [1.0, 2.03], [1.0, 2.0], 2e-2)
