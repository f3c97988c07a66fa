"""Per-channel balance scale (calibration statistic of the MXFP4 path).

Test infrastructure only (see ``oracle/__init__``).

Definition ("MACaQ", paper 2611.10649, "Core method" step (i) and "Method
steps" step 1): t_j = (sigma^W_j)**alpha / (rms^x_j)**(1 - alpha) with
alpha = 0.75; activations are multiplied by t_j, weight columns divided by
t_j, and t is "range clipped" for numerical stability.

Readings taken where the page is silent: sigma^W_j is the population
standard deviation of input column j of W [N, K] over its N rows;
rms^x_j = sqrt(mean_t X[t, j]**2) over the calibration rows; each factor is
floored at 1e-12 and t is clipped to [2**-16, 2**16].  Everything is float64;
the hot path receives t32 = fl32(t) for activations and u32 = fl32(1/t) for
weights.
"""

from __future__ import annotations

import numpy as np

ALPHA = 0.75
FLOOR = 1e-12
T_MIN = 2.0 ** -16
T_MAX = 2.0 ** 16


def balance_scale(w: np.ndarray, x: np.ndarray, alpha: float = ALPHA):
    """Return ``(t64, t32, u32)`` for weights ``w`` [N, K] and calibration
    activations ``x`` [M, K] (any real dtype, widened to float64)."""
    w = np.asarray(w, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    assert w.shape[1] == x.shape[1]
    sigma = w.std(axis=0, ddof=0)
    rms = np.sqrt((x * x).mean(axis=0))
    t = np.maximum(sigma, FLOOR) ** alpha / np.maximum(rms, FLOOR) ** (1.0 - alpha)
    t = np.clip(t, T_MIN, T_MAX)
    return t, t.astype(np.float32), (1.0 / t).astype(np.float32)
