"""Comparison metrics.  TEST INFRASTRUCTURE ONLY.

[DG-FP8] "精度与吞吐的平衡点": the DeepGEMM tests accept an FP8 x FP8 result whose
``calc_diff`` against the reference is below 0.001 (0.01 with one FP4 side).
The page names the function but not its formula; the reading used here is
    diff = 1 - 2 * sum(x*y) / sum(x*x + y*y)
(0 for identical vectors, 2 for x = -y; 0 when both are all-zero), computed
in float64 over the valid rows only.  A per-element bound is checked as well:
    |x - y| <= 2e-2 * |y| + 1e-2 * rms(y).
"""

from __future__ import annotations

import numpy as np


def calc_diff(x, y) -> float:
    """Pinned by closed forms: diff(x, x) = 0, diff(x, -x) = 2, diff(x, c x) = (1-c)^2/(1+c^2)."""
    x = np.asarray(x, dtype=np.float64).reshape(-1)
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    den = float(np.sum(x * x + y * y))
    if den == 0.0:
        return 0.0
    return 1.0 - 2.0 * float(np.sum(x * y)) / den


def elementwise_excess(x, y_ref, rel: float = 2e-2, abs_rms: float = 1e-2) -> float:
    """max over elements of |x - y| - (rel*|y| + abs_rms*rms(y)); <= 0 means within bound."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(y * y))) if y.size else 0.0
    if x.size == 0:
        return -1.0
    return float(np.max(np.abs(x - y) - (rel * np.abs(y) + abs_rms * rms)))


def elementwise_ok(x, y_ref, rel: float = 2e-2, abs_rms: float = 1e-2) -> bool:
    return elementwise_excess(x, y_ref, rel, abs_rms) <= 0.0
