"""Weighted combine back to token order.  TEST INFRASTRUCTURE ONLY.

[GEMM-modes] sec. 4.4 and 4.6: z_t = sum_r p[t, r] * y_packed[output_index[t, r]],
reading only rows named by output_index (padding rows have none).  [CuTeDSL]:
the combine accumulates the gathered rows in registers.  Slots whose
output_index is -1 (dropped or invalid routes) contribute nothing.
Weights are used as given (no renormalisation).
"""

from __future__ import annotations

import numpy as np


def combine(y: np.ndarray, output_index: np.ndarray, topk_weights: np.ndarray) -> np.ndarray:
    """float64 [T, N]; y is float64 [rows, N] (or anything convertible).

    Pinned by: the page's worked example (z_0 combines packed rows 0 and 256
    with weights 0.70 and 0.30 in the aligned layout) and exact rational
    brute force.
    """
    y = np.asarray(y, dtype=np.float64)
    T, k = output_index.shape
    N = y.shape[1]
    z = np.zeros((T, N), dtype=np.float64)
    for t in range(T):
        for r in range(k):
            p = int(output_index[t, r])
            if p < 0:
                continue
            z[t] += float(topk_weights[t, r]) * y[p]
    return z
