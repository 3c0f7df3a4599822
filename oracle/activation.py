"""SwiGLU between the up- and down-projection, and its 1x128 FP8 requantisation.
TEST INFRASTRUCTURE ONLY (see package header).

The pages feed the grouped GEMM with a fused gate+up weight (the DeepSeek-V3
expert's up-projection has 2 x 2048 output columns) and list activation
kernels among the MoE building blocks ([CuTeDSL]: the kernel library holds
activation functions next to the MoE dispatch/combine), but print no formula.
Readings taken (listed in the design notes):
  * SwiGLU(gate, up) = silu(gate) * up with silu(x) = x / (1 + exp(-x)),
    elementwise; the up-projection's N = 2I columns hold gate in columns
    0 .. I-1 and up in columns I .. 2I-1 (the order of the fused gate+up
    weight);
  * the result is requantised for the down-projection exactly as activations
    are ([DG-FP8] "补偿机制一"): per row and 128-column block, scale = the
    smallest power of two 2^e with amax <= 448 * 2^e, codes = E4M3 RNE of
    h * 2^-e.  h is quantised as computed, with no bf16 rounding in between.

The oracle evaluates h in float64 and quantises the float64 values.
"""

from __future__ import annotations

import numpy as np

from .quant import BLOCK, _quant_blocks


def silu(x) -> np.ndarray:
    """x / (1 + exp(-x)) in float64 (exp overflow for x < -709 gives -0.0 / 0.0, never NaN).

    Pinned by: closed forms silu(0) = 0, silu(ln 3) = 0.75 ln 3, silu(-ln 3) = -0.25 ln 3; the identity
    silu(x) - silu(-x) = x; 40-digit decimal evaluation of random arguments.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(gate_up) -> np.ndarray:
    """float64 [rows, I] = silu(gate) * up for gate_up float64 [rows, 2I] (gate first, then up)."""
    gu = np.asarray(gate_up, dtype=np.float64)
    rows, n2 = gu.shape
    if n2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    i = n2 // 2
    return silu(gu[:, :i]) * gu[:, i:]


def quant_act_values(x) -> tuple[np.ndarray, np.ndarray]:
    """1x128 FP8 quantisation of float64 rows (the activation rule of quant_act, on values instead of bf16).

    Returns (codes uint8 [rows, K], sf float32 [rows, K/128]).
    Pinned by: equality with quant_act on bf16-valued inputs, and the pow2 and error-bound properties.
    """
    x = np.asarray(x, dtype=np.float64)
    rows, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    amax = np.abs(x.reshape(rows, K // BLOCK, BLOCK)).max(axis=2)
    return _quant_blocks(x, amax, lambda s: np.repeat(s, BLOCK, axis=1))


def swiglu_quant(gate_up) -> tuple[np.ndarray, np.ndarray]:
    """(codes uint8 [rows, I], sf float32 [rows, I/128]) of SwiGLU(gate_up) requantised per 1x128 block."""
    return quant_act_values(swiglu(gate_up))
