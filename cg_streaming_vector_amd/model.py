"""The streaming performance model of "Portable high-order finite element
kernels I: Streaming Operations" (arXiv 2009.10917, performance model
section): T(B) = T0 + B / W_max (eq. 8), effective bandwidth
W_eff(B) = B / T(B) (eq. 9), and the Fischer-Brown point B_0.8 at which
W_eff = 0.8 W_max, B_0.8 = 4 T0 W_max (eq. 10).

The pages fit the model "to the measured bandwidth" without naming a method.
Here the fit minimises the relative error of the modelled bandwidth,
sum_i ((W_eff(B_i) - W_i) / W_i)^2 to first order, which is the relative error
of the modelled time, sum_i ((T0 + s B_i - T_i) / T_i)^2 with s = 1/W_max: a
weighted linear least-squares problem in (T0, s), solved in closed form.
"""
from __future__ import annotations

import numpy as np


def t_model(B, T0, W_max):
    """Eq. 8: time to stream B bytes."""
    return T0 + np.asarray(B, dtype=np.float64) / W_max


def w_eff(B, T0, W_max):
    """Eq. 9: effective bandwidth when streaming B bytes."""
    B = np.asarray(B, dtype=np.float64)
    return B / t_model(B, T0, W_max)


def fischer_brown(T0, W_max, frac=0.8):
    """Bytes at which W_eff reaches frac * W_max: frac/(1-frac) T0 W_max
    (eq. 10 for frac = 0.8: 4 T0 W_max)."""
    return frac / (1.0 - frac) * T0 * W_max


def fit_streaming_model(B, T):
    """Fit eq. 8 to measured (bytes, seconds) pairs.

    Returns T0 [s], W_max [bytes/s], W_max_GBps, B_0.8 [bytes] and the R^2 of
    the modelled bandwidth against the measured bandwidth."""
    B = np.asarray(B, dtype=np.float64)
    T = np.asarray(T, dtype=np.float64)
    if B.size < 2 or np.any(T <= 0):
        raise ValueError("need at least two positive timings")
    w = 1.0 / T
    A = np.stack([w, B * w], axis=1)
    (T0, s), *_ = np.linalg.lstsq(A, np.ones_like(T), rcond=None)
    if s <= 0:
        raise ValueError("fitted bandwidth is not positive")
    W_max = 1.0 / s
    W = B / T
    Wm = w_eff(B, T0, W_max)
    ss_res = float(np.sum((W - Wm) ** 2))
    ss_tot = float(np.sum((W - W.mean()) ** 2))
    r2 = 1.0 - ss_res / ss_tot if ss_tot > 0 else 1.0
    return {"T0_s": float(T0), "W_max": float(W_max), "W_max_GBps": float(W_max / 1e9),
            "B_08_bytes": float(fischer_brown(T0, W_max)), "r2_bandwidth": r2}
