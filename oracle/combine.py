"""Weighted combine back to token order.  TEST INFRASTRUCTURE ONLY.

[GEMM-modes] sec. 4.4 and 4.6: z_t = sum_r p[t, r] * y_packed[output_index[t, r]],
reading only rows named by output_index (padding rows have none).  [CuTeDSL]:
the combine accumulates the gathered rows in registers.  Slots whose
output_index is -1 (dropped or invalid routes), or names no row of y,
contribute nothing.
Weights are used as given (no renormalisation).

Two forms:
  combine       the plain sum in float64 (the value the method approximates);
  combine_fp32  the same sum as the path defines its precision (reading A13 of
                the pages' open points: an fp32 fused multiply-add per slot in
                slot order r = 0..k-1 starting from +0, then one round to
                nearest even to bf16).  Every fma is evaluated exactly and
                rounded once to fp32, so the result is a unique bit pattern.
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
            if p < 0 or p >= y.shape[0]:
                continue
            z[t] += float(topk_weights[t, r]) * y[p]
    return z


def _fma_f32(w: np.ndarray, y: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """fp32 fused multiply-add RN(w*y + acc) for fp32 w and acc and bf16-valued y, elementwise.

    w*y has at most 24 + 8 significant bits, so the float64 product is exact.
    The float64 sum s = p + acc is exact up to the error term e of the
    two-sum (p + acc = s + e exactly, |e| <= half an ulp of s in float64).  s
    rounds to the same fp32 as s + e unless s is exactly halfway between two
    fp32 neighbours (every other float64 lies at least one float64 ulp from a
    halfway point); then the sign of e decides which neighbour is nearer.
    """
    p = w.astype(np.float64) * y.astype(np.float64)
    a = acc.astype(np.float64)
    s = p + a
    bp = s - p
    ap = s - bp
    e = (p - ap) + (a - bp)
    r = s.astype(np.float32).astype(np.float64)      # round to nearest even
    other = 2.0 * s - r                                 # the other neighbour when s is halfway
    halfway = (s != r) & (other.astype(np.float32).astype(np.float64) == other)
    take_other = halfway & (e != 0) & (np.sign(e) == np.sign(other - r))
    return np.where(take_other, other, r).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def combine_fp32(y_bits: np.ndarray, output_index: np.ndarray, topk_weights: np.ndarray) -> np.ndarray:
    """bf16 bit patterns uint16 [T, N] of the fp32 fma-chain combine (reading A13).

    y_bits: uint16 bf16 patterns [rows, N]; topk_weights: float32 [T, k] (used as given).
    Slots with output_index < 0 or >= rows are skipped.

    Pinned by: exact rational evaluation (fractions.Fraction, rounded to fp32
    after every step) on small cases; equality with plain float32 arithmetic
    where every product is exact in fp32; and the error bound against combine().
    """
    y_bits = np.asarray(y_bits, dtype=np.uint16)
    rows, N = y_bits.shape
    yv = (y_bits.astype(np.uint32) << 16).view(np.float32)
    w = np.asarray(topk_weights, dtype=np.float32)
    T, k = output_index.shape
    acc = np.zeros((T, N), dtype=np.float32)
    for r in range(k):
        p = np.asarray(output_index[:, r], dtype=np.int64)
        ok = (p >= 0) & (p < rows)
        if not ok.any():
            continue
        nxt = _fma_f32(np.broadcast_to(w[ok, r][:, None], (int(ok.sum()), N)), yv[p[ok]], acc[ok])
        acc[ok] = nxt
    return f32_to_bf16_bits(acc)
