"""Negative probes of the comparison rules (CPU): each must reject planted
bad evidence (the rejection probes of page "Scale coverage exposes a
remaining GEMM gap", section "Measurement contract and evidence")."""
import numpy as np
import pytest

from tests.compare import bitexact_mismatches, rel_rms


def _ref():
    rng = np.random.default_rng(5)
    return rng.integers(-50, 50, (33, 17)).astype(np.float64)


def test_equal_passes():
    r = _ref()
    assert bitexact_mismatches(r.astype(np.float32), r) == 0
    assert rel_rms(r.astype(np.float32), r) == 0.0


def test_one_ulp_is_caught():
    r = _ref()
    g = r.astype(np.float32)
    g.view(np.uint32)[3, 4] += 1
    assert bitexact_mismatches(g, r) == 1
    assert rel_rms(g, r) > 0.0


def test_negative_zero_is_caught():
    r = np.zeros((4, 4))
    g = r.astype(np.float32)
    g[1, 1] = -0.0
    assert bitexact_mismatches(g, r) == 1


def test_nan_is_caught():
    r = _ref()
    g = r.astype(np.float32)
    g[0, 0] = np.nan
    assert bitexact_mismatches(g, r) == 1
    assert rel_rms(g, r) == float("inf")


def test_missing_element_is_caught():
    r = _ref()
    g = r.astype(np.float32)[:, :-1]
    with pytest.raises(ValueError):
        bitexact_mismatches(g, r)
    with pytest.raises(ValueError):
        rel_rms(g, r)


def test_rel_rms_scale():
    r = _ref() + 0.5
    g = (r * (1 + 1e-3)).astype(np.float32)
    assert 5e-4 < rel_rms(g, r) < 2e-3
