"""The streaming model T(B) = T0 + B/W_max (arXiv 2009.10917, eqs. 8-10)."""
import numpy as np
import pytest

from cg_streaming_vector_amd.model import fischer_brown, fit_streaming_model, t_model, w_eff


def test_fischer_brown_is_eq10():
    T0, W = 4.2e-6, 6.1e12
    B = fischer_brown(T0, W)
    assert B == pytest.approx(4 * T0 * W, rel=1e-15)
    # by definition W_eff(B_0.8) = 0.8 W_max
    assert w_eff(B, T0, W) == pytest.approx(0.8 * W, rel=1e-14)
    # and W_eff is below 0.8 W_max just before, above just after
    assert w_eff(0.99 * B, T0, W) < 0.8 * W < w_eff(1.01 * B, T0, W)


@pytest.mark.parametrize("T0,W", [(3e-6, 5.5e12), (1.2e-5, 2.0e11), (0.0, 1e12)])
def test_fit_recovers_parameters(T0, W):
    B = 16.0 * 2.0 ** np.arange(10, 29)
    T = t_model(B, T0, W)
    f = fit_streaming_model(B, T)
    assert f["T0_s"] == pytest.approx(T0, abs=1e-12)
    assert f["W_max"] == pytest.approx(W, rel=1e-9)
    assert f["B_08_bytes"] == pytest.approx(4 * T0 * W, rel=1e-6, abs=1e-3)
    assert f["r2_bandwidth"] == pytest.approx(1.0, abs=1e-12)


def test_fit_with_noise_is_close():
    rng = np.random.default_rng(5)
    B = 24.0 * 2.0 ** np.arange(10, 29)
    T = t_model(B, 4e-6, 6e12) * (1 + 0.02 * rng.standard_normal(B.size))
    f = fit_streaming_model(B, T)
    assert f["T0_s"] == pytest.approx(4e-6, rel=0.1)
    assert f["W_max"] == pytest.approx(6e12, rel=0.05)
    assert f["r2_bandwidth"] > 0.95


def test_fit_rejects_bad_input():
    with pytest.raises(ValueError):
        fit_streaming_model([1.0], [1.0])
    with pytest.raises(ValueError):
        fit_streaming_model([1.0, 2.0], [0.0, 1.0])
