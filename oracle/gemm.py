"""Grouped GEMM over packed expert segments.  TEST INFRASTRUCTURE ONLY.

[GEMM-modes] sec. 4.1/4.4: a grouped GEMM is P independent problems and equals
P single GEMMs; expert e computes Y_e = X_e W_e^T with W_e in R^{N x K} (both
operands K-contiguous, "NT").  Sec. 4.6: every packed row uses the weights of
its expert and rows are independent along K, so padding rows never mix into
valid ones.  [AsymGEMM] "API Reference": FP8 operands come as (data, scale)
pairs, outputs are bf16.  [DG-FP8]: FP32 accumulation with fine-grained scales.

The oracle evaluates the exact block-scaled sum in float64:
    D[p, n] = sum_k (dec(a[p,k]) * sa[p, k/128]) * (dec(w[e,n,k]) * sw[e, n/128, k/128])
Every product is exact in float64 (<= 4+4 significant bits times powers of
two) and each 128-block partial sum is exact; the cross-block float64 sum is
within a few ulps of the exact value.  Output rows that belong to no valid
assignment are NaN (never compared).

INT4 ([MatMulNBits] sec. 2):  D[p, n] = sum_k a[p,k] * (q[e,n,k] - 8) * s[e, n, k/128].

FP8 x FP4 ([AsymGEMM] "API Reference", FP4 grouped GEMMs; [CuTeDSL] MXFP4 block scaling;
[DG-FP8] "精度与吞吐的平衡点": one FP4 side is held to calc_diff < 0.01):
    D[p, n] = sum_k (dec8(a[p,k]) * sa[p, k/128]) * (dec4(w[e,n,k]) * 2^(sw[e,n,k/32] - 127)).

INT8 ([AsymGEMM] "API Reference", INT8 m_grouped contiguous / masked with the (1, 1, 128) recipe):
    D[p, n] = sum_k (a[p,k] * sa[p, k/128]) * (w[e,n,k] * sw[e, n, k/128])   with int8 codes.
Each 128-block's integer sum is exact, and so is every product with the two fp32 scales in float64.

BF16 ([AsymGEMM] "API Reference", BF16 m_grouped contiguous / masked; [GEMM-modes]
sec. 4.6, the BF16 contiguous grouped GEMM SGLang calls):
    D[p, n] = sum_k a[p,k] * w[e,n,k]   with bf16 operands, in float64.
Every product of two bf16 values is exact in float64 (8 + 8 significant bits)
and sums of them stay exact while the exponent range of a row is modest, so
the result is the exact value for all practical purposes.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64
from .quant import dequant_act, dequant_int8, dequant_weight_fp4, dequant_weight_fp8, dequant_weight_int4


def segments(counts, seg_offsets):
    """[(expert, first_row, n_rows)] for every expert with rows."""
    return [(e, int(seg_offsets[e]), int(counts[e])) for e in range(len(counts)) if int(counts[e]) > 0]


def grouped_gemm_fp8(a_codes, sfa, w_codes, sfw, counts, seg_offsets, rows_out=None,
                     experts=None):
    """FP8 block-scaled grouped GEMM in float64.

    a_codes uint8 [rows, K], sfa float32 [rows, K/128];
    w_codes uint8 [E, N, K], sfw float32 [E, N/128, K/128];
    segment e = rows [seg_offsets[e], seg_offsets[e] + counts[e]).
    ``experts`` (optional) restricts the work to those experts; when given,
    w_codes/sfw may hold just those experts in the same order.
    Returns float64 [rows_out, N] (NaN outside valid rows).

    Pinned by: exact rational brute force on tiny shapes, closed-form one-hot
    and small-integer cases, scale invariance, per-expert single-GEMM equivalence.
    """
    rows = a_codes.shape[0] if rows_out is None else rows_out
    E_all = len(counts)
    N = w_codes.shape[-2]
    out = np.full((rows, N), np.nan, dtype=np.float64)
    sel = range(E_all) if experts is None else list(experts)
    for j, e in enumerate(sel):
        c = int(counts[e])
        if c <= 0:
            continue
        wi = e if experts is None else j
        p0 = int(seg_offsets[e])
        a = dequant_act(a_codes[p0:p0 + c], sfa[p0:p0 + c])
        w = dequant_weight_fp8(w_codes[wi], sfw[wi])
        out[p0:p0 + c] = a @ w.T
    return out


def grouped_gemm_bf16(a_bits, w_bits, counts, seg_offsets, rows_out=None, experts=None):
    """BF16 grouped GEMM in float64.

    a_bits uint16 [rows, K] bf16; w_bits uint16 [E, N, K] bf16.
    Returns float64 [rows_out, N] (NaN outside valid rows).

    Pinned by: exact rational brute force, small-integer and one-hot cases, per-expert single-GEMM
    equivalence.
    """
    rows = a_bits.shape[0] if rows_out is None else rows_out
    E_all = len(counts)
    N = w_bits.shape[-2]
    out = np.full((rows, N), np.nan, dtype=np.float64)
    sel = range(E_all) if experts is None else list(experts)
    for j, e in enumerate(sel):
        c = int(counts[e])
        if c <= 0:
            continue
        wi = e if experts is None else j
        p0 = int(seg_offsets[e])
        a = bf16_bits_to_f64(a_bits[p0:p0 + c])
        w = bf16_bits_to_f64(w_bits[wi])
        out[p0:p0 + c] = a @ w.T
    return out


def grouped_gemm_fp8_fp4(a_codes, sfa, w4, sw, counts, seg_offsets, rows_out=None, experts=None):
    """FP8 activations x MXFP4 weights grouped GEMM in float64.

        D[p, n] = sum_k (dec8(a[p,k]) * sa[p, k/128]) * (dec4(w[e,n,k]) * 2^(sw[e, n, k/32] - 127))

    a_codes uint8 [rows, K] E4M3, sfa float32 [rows, K/128]; w4 uint8 [E, N, K/2] E2M1 pairs (even k low),
    sw uint8 [E, N, K/32] E8M0.  Every product is exact in float64 and so is each 32-block partial sum.
    Returns float64 [rows_out, N] (NaN outside valid rows).

    Pinned by: exact rational brute force, small-integer codes vs integer matmul, one-hot rows, scale
    invariance, per-expert single-GEMM equivalence.
    """
    rows = a_codes.shape[0] if rows_out is None else rows_out
    E_all = len(counts)
    N = w4.shape[-2]
    out = np.full((rows, N), np.nan, dtype=np.float64)
    sel = range(E_all) if experts is None else list(experts)
    for j, e in enumerate(sel):
        c = int(counts[e])
        if c <= 0:
            continue
        wi = e if experts is None else j
        p0 = int(seg_offsets[e])
        a = dequant_act(a_codes[p0:p0 + c], sfa[p0:p0 + c])
        out[p0:p0 + c] = a @ dequant_weight_fp4(w4[wi], sw[wi]).T
    return out


def grouped_gemm_int4(a_bits, w_q4, s16_bits, counts, seg_offsets, rows_out=None,
                      experts=None):
    """INT4 weight-only grouped GEMM in float64.

    a_bits uint16 [rows, K] bf16; w_q4 uint8 [E, N, K/2]; s16_bits uint16 [E, N, K/128].
    Returns float64 [rows_out, N] (NaN outside valid rows).
    """
    rows = a_bits.shape[0] if rows_out is None else rows_out
    E_all = len(counts)
    N = w_q4.shape[-2]
    out = np.full((rows, N), np.nan, dtype=np.float64)
    sel = range(E_all) if experts is None else list(experts)
    for j, e in enumerate(sel):
        c = int(counts[e])
        if c <= 0:
            continue
        wi = e if experts is None else j
        p0 = int(seg_offsets[e])
        a = bf16_bits_to_f64(a_bits[p0:p0 + c])
        w = dequant_weight_int4(w_q4[wi], s16_bits[wi])
        out[p0:p0 + c] = a @ w.T
    return out


def grouped_gemm_int8(a_q, sa, w_q, sw, counts, seg_offsets, rows_out=None, experts=None):
    """INT8 (1, 1, 128) grouped GEMM in float64.

    a_q int8 [rows, K], sa float32 [rows, K/128]; w_q int8 [E, N, K], sw float32 [E, N, K/128];
    segments and ``experts`` as for grouped_gemm_fp8.  Returns float64 [rows_out, N] (NaN outside valid rows).

    Pinned by: exact rational brute force on tiny shapes, integer codes with unit scales against an integer
    matmul, per-row and per-channel scale factoring, per-expert single-GEMM equivalence, a swapped-scale
    mistake caught.
    """
    rows = a_q.shape[0] if rows_out is None else rows_out
    N = w_q.shape[-2]
    out = np.full((rows, N), np.nan, dtype=np.float64)
    sel = range(len(counts)) if experts is None else list(experts)
    for j, e in enumerate(sel):
        c = int(counts[e])
        if c <= 0:
            continue
        wi = e if experts is None else j
        p0 = int(seg_offsets[e])
        out[p0:p0 + c] = dequant_int8(a_q[p0:p0 + c], sa[p0:p0 + c]) @ dequant_int8(w_q[wi], sw[wi]).T
    return out
