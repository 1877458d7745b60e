"""The parity metric itself (host logic, no GPU): assert_close applies both the
normwise bound and the elementwise bound |got - ref| <= tol |ref| + tol rms(ref),
so an element much smaller than the tensor's maximum cannot be badly wrong and
still pass."""
import numpy as np
import pytest

from gpu_helpers import assert_close, elementwise, rel_err


def test_normwise_passes_but_elementwise_catches_a_small_element():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(10000)
    ref[17] = 1e-3 * ref.std()          # a small element...
    got = ref.copy()
    got[17] = -ref[17] * 40             # ...that is badly wrong
    assert rel_err(got, ref) < 2e-2     # invisible to the normwise metric
    with pytest.raises(AssertionError, match="elementwise"):
        assert_close("t", got, ref, 2e-2)


def test_rounding_sized_errors_pass():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal(10000)
    got = ref * (1 + 2.0 ** -9 * rng.uniform(-1, 1, ref.shape))  # bf16-size rounding
    assert_close("t", got, ref, 2e-2)


def test_worst_element_and_rel_l2_reported():
    ref = np.array([1.0, 2.0, -4.0, 0.5])
    got = np.array([1.0, 2.0, -4.1, 0.5])
    el = elementwise(got, ref, 1e-2)
    assert el["worst"][0] == (2,)
    assert abs(el["rel_l2"] - 0.1 / np.sqrt(1 + 4 + 16 + 0.25)) < 1e-12
    assert el["ratio"] > 1.0


def test_nan_mismatch_fails():
    with pytest.raises(AssertionError):
        assert_close("t", np.array([1.0, np.nan]), np.array([1.0, 2.0]), 1e-2)
