"""FP8 block quantisation with power-of-two scales, and the 4-bit weight format.
TEST INFRASTRUCTURE ONLY (see package header).

FP8 ([DG-FP8] "补偿机制一", [AsymGEMM] "API Reference"):
  * recipe (gran_m, gran_n, gran_k) = (1, 128, 128): activations share one
    scale per 1x128 block along K, weights one per 128x128 block;
  * every scale is an exact power of two (fp32 bit pattern 0.eeeeeeee.000...0),
    so applying it is an exponent shift with no rounding;
  * the scale is chosen by rounding amax/448 UP to a power of two (the article
    names the helper ``ceil_to_ue8m0``), so no scaled value exceeds 448 and no
    saturation is needed.  Reading taken: scale = 2^e with e the smallest
    integer such that amax <= 448 * 2^e; e clamped to [-126, 127]; amax == 0
    gives scale 1.
  * codes = round-to-nearest-even E4M3 of x * 2^-e (exact multiply).

INT4 ([MatMulNBits] sec. 2 "Weight Format"): each output row n stores K/2 bytes,
two 4-bit weights per byte (the low nibble holds the even k), one scale per
128-element block along K, values 0..15 meaning (q - 8) * scale.  The page does
not say how the scales were chosen (weights are quantised offline).  Reading
taken for the synthetic weights: s = fp16(fp32(amax) / 7) per (n, block), with
amax == 0 giving s = 1, an underflow to 0 giving the smallest fp16 subnormal,
and q = clip(rne(w / s) + 8, 0, 15), where the divisions are done in fp32
because they decide integer codes and the GPU kernel decides them in fp32.
"""

from __future__ import annotations

import math

import numpy as np

from .formats import (E2M1_MAX, E4M3_MAX, bf16_bits_to_f64, e2m1_decode_table, e2m1_encode, e4m3_decode_table,
                      e4m3_encode, e8m0_value, fp16_bits_to_f64)

BLOCK = 128
EXP_MIN, EXP_MAX = -126, 127


def pow2_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-126, 127]; 0 for amax == 0.

    Written as the definition: start near log2(amax/448) and step until the
    defining inequality holds and fails one step below.  All comparisons are
    exact (ldexp of 448 is exact in float64).

    Pinned by: minimality (448*2^(e-1) < amax <= 448*2^e) on random and edge
    values, and equality with ceil(log2(fp32(amax/448))) for every positive bf16.
    """
    amax = float(amax)
    if amax < 0 or math.isnan(amax):
        raise ValueError("amax must be a non-negative number")
    if amax == 0.0:
        return 0
    e = int(math.floor(math.log2(amax / E4M3_MAX)))
    while amax > math.ldexp(E4M3_MAX, e):
        e += 1
    while amax <= math.ldexp(E4M3_MAX, e - 1):
        e -= 1
    return min(max(e, EXP_MIN), EXP_MAX)


def pow2_exponents(amax: np.ndarray) -> np.ndarray:
    """Element-wise pow2_exponent over an array (same definition, looped)."""
    a = np.asarray(amax, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.int32)
    fa, fo = a.reshape(-1), out.reshape(-1)
    for i in range(fa.size):
        fo[i] = pow2_exponent(fa[i])
    return out


def _quant_blocks(xf: np.ndarray, amax: np.ndarray, scale_shape_expand):
    e = pow2_exponents(amax)
    scale = np.ldexp(np.ones(e.shape), e)
    s_full = scale_shape_expand(scale)
    codes = e4m3_encode(xf / s_full)  # division by a power of two: exact
    return codes, scale.astype(np.float32)


def quant_act(x_bits: np.ndarray):
    """1x128 activation quantisation of bf16 rows.

    x_bits: uint16 [rows, K] bf16 patterns, K % 128 == 0.
    Returns (codes uint8 [rows, K], sf float32 [rows, K/128]).
    Pinned by: pow2 invariants, rescale invariance, encoder pins, error bound.
    """
    x = bf16_bits_to_f64(x_bits)
    rows, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    kb = K // BLOCK
    amax = np.abs(x.reshape(rows, kb, BLOCK)).max(axis=2)
    return _quant_blocks(x, amax, lambda s: np.repeat(s, BLOCK, axis=1))


def quant_weight_fp8(w_bits: np.ndarray):
    """128x128 weight quantisation of bf16 expert weights.

    w_bits: uint16 [E, N, K]; N, K multiples of 128.
    Returns (codes uint8 [E, N, K], sfw float32 [E, N/128, K/128]).
    """
    w = bf16_bits_to_f64(w_bits)
    E, N, K = w.shape
    if N % BLOCK or K % BLOCK:
        raise ValueError("N and K must be multiples of 128")
    nb, kb = N // BLOCK, K // BLOCK
    amax = np.abs(w.reshape(E, nb, BLOCK, kb, BLOCK)).max(axis=(2, 4))

    def expand(s):
        return np.repeat(np.repeat(s, BLOCK, axis=1), BLOCK, axis=2)

    return _quant_blocks(w, amax, expand)


def dequant_act(codes: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """float64 [rows, K] = decode(codes) * scale of the code's 1x128 block."""
    tab = e4m3_decode_table()
    return tab[codes] * np.repeat(sf.astype(np.float64), BLOCK, axis=1)


def dequant_weight_fp8(codes: np.ndarray, sfw: np.ndarray) -> np.ndarray:
    """float64 [..., N, K] = decode(codes) * scale of the code's 128x128 block."""
    tab = e4m3_decode_table()
    s = np.repeat(np.repeat(sfw.astype(np.float64), BLOCK, axis=-2), BLOCK, axis=-1)
    return tab[codes] * s


def quant_weight_int4(w_bits: np.ndarray):
    """Group-128 4-bit weight quantisation (reading stated in the module header).

    w_bits: uint16 [E, N, K] bf16 patterns.
    Returns (q4 uint8 [E, N, K/2] with the even k in the low nibble,
             s16 uint16 [E, N, K/128] fp16 bit patterns).
    Pinned by: range/round-trip properties and exact integer cases (tests).
    """
    w32 = bf16_bits_to_f64(w_bits).astype(np.float32)  # exact
    E, N, K = w32.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    g = K // BLOCK
    amax = np.abs(w32.reshape(E, N, g, BLOCK)).max(axis=3)
    s32 = (amax / np.float32(7.0)).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    s16 = np.where(amax == 0, np.float16(1.0), s16)
    s16 = np.where((amax > 0) & (s16 == 0), np.float16(2.0 ** -24), s16)
    s16 = np.minimum(s16, np.float16(65504.0)).astype(np.float16)
    s_full = np.repeat(s16.astype(np.float32), BLOCK, axis=2)
    q = np.rint(w32 / s_full).astype(np.float32)  # fp32 division, ties to even
    q = np.clip(q + 8.0, 0.0, 15.0).astype(np.uint8)
    q4 = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    return q4, s16.view(np.uint16)


def unpack_int4(q4: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> uint8 [..., K]: element 2j is the low nibble of byte j."""
    q4 = np.asarray(q4, dtype=np.uint8)
    out = np.empty(q4.shape[:-1] + (q4.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = q4 & 0x0F
    out[..., 1::2] = q4 >> 4
    return out


def dequant_weight_int4(q4: np.ndarray, s16_bits: np.ndarray) -> np.ndarray:
    """float64 [..., N, K] = (q - 8) * scale of the weight's 128-group."""
    q = unpack_int4(q4).astype(np.float64)
    s = np.repeat(fp16_bits_to_f64(s16_bits), BLOCK, axis=-1)
    return (q - 8.0) * s


# ------------------------------------------------------------------------------------- FP4 (MXFP4) weights --
FP4_BLOCK = 32
E8M0_MIN, E8M0_MAX = -127, 127


def pow2_exponent_e2m1(amax: float) -> int:
    """Smallest integer e with amax <= 6 * 2^e, clamped to [-127, 127]; 0 for amax == 0 (the FP8 rule with the
    E2M1 maximum 6).  Pinned by: minimality on random and edge values."""
    amax = float(amax)
    if amax < 0 or math.isnan(amax):
        raise ValueError("amax must be a non-negative number")
    if amax == 0.0:
        return 0
    e = int(math.floor(math.log2(amax / E2M1_MAX)))
    while amax > math.ldexp(E2M1_MAX, e):
        e += 1
    while amax <= math.ldexp(E2M1_MAX, e - 1):
        e -= 1
    return min(max(e, E8M0_MIN), E8M0_MAX)


def quant_weight_fp4(w_bits: np.ndarray):
    """MXFP4 weight quantisation: one power-of-two scale per 32 consecutive K values of an output column.

    Reading taken (the pages give the FP4 element format and block scaling, not the offline rule): the scale is
    the smallest power of two 2^e with amax <= 6 * 2^e (rounded up, as the FP8 rule), stored as the E8M0 byte
    e + 127; codes = E2M1 RNE of w * 2^-e (exact multiply), two per byte, the even k in the low nibble.
    w_bits: uint16 [E, N, K] bf16, K % 128 == 0.
    Returns (w4 uint8 [E, N, K/2], sw uint8 [E, N, K/32]).
    Pinned by: the scale rule's minimality and amax bound, the E2M1 error bound, rescale invariance.
    """
    w = bf16_bits_to_f64(w_bits)
    E, N, K = w.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    nb = K // FP4_BLOCK
    amax = np.abs(w.reshape(E, N, nb, FP4_BLOCK)).max(axis=3)
    e = np.vectorize(pow2_exponent_e2m1, otypes=[np.int64])(amax) if amax.size else amax.astype(np.int64)
    scaled = w / np.repeat(np.ldexp(np.ones(e.shape), e), FP4_BLOCK, axis=2)
    codes = e2m1_encode(scaled)
    w4 = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return w4, (e + 127).astype(np.uint8)


def dequant_weight_fp4(w4: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """float64 [..., N, K] = decode(code) * 2^(sw - 127) of the code's 32-block."""
    codes = unpack_int4(w4)
    return e2m1_decode_table()[codes] * np.repeat(e8m0_value(sw), FP4_BLOCK, axis=-1)


# ------------------------------------------------------------------------------------------ INT8 (1, 1, 128) --
INT8_MAX = 127


def quant_int8(x_bits: np.ndarray):
    """INT8 (1, 1, 128) block quantisation ([AsymGEMM] "API Reference", INT8 asymmetric GEMM: (int8 data, fp32
    scale) pairs with one scale per row and 128-element block along K, per token for activations and per output
    channel for weights).  The page gives no rule for choosing the scale; reading taken: symmetric,
    s = fp32(amax) / 127 (fp32 division, round to nearest), and q = clip(rne(x / s), -127, 127) with the
    division in fp32 (it decides an integer code, and the GPU kernel decides it in fp32); amax == 0 gives s = 1
    and q = 0.

    x_bits: uint16 [..., K] bf16 patterns (rows: tokens, or the N rows of each expert's weight).
    Returns (q int8 [..., K], s float32 [..., K/128]).
    Pinned by: an exact rational evaluation of every step (fp32 rounding written out from its definition) on
    random and edge blocks; |q| <= 127 with the block's largest magnitude at +-127; the error bound
    |x - q s| <= s / 2 (plus the fp32 rounding of x / s); sign symmetry; 2^j x giving the same codes and
    scales 2^j s.
    """
    x32 = bf16_bits_to_f64(x_bits).astype(np.float32)  # exact
    K = x32.shape[-1]
    if K % BLOCK:
        raise ValueError("K must be a multiple of 128")
    xb = x32.reshape(x32.shape[:-1] + (K // BLOCK, BLOCK))
    amax = np.abs(xb).max(axis=-1)
    s = np.where(amax > 0, amax / np.float32(INT8_MAX), np.float32(1.0)).astype(np.float32)
    q = np.rint(xb / s[..., None]).astype(np.float32)  # fp32 division, ties to even
    q = np.clip(q, -INT8_MAX, INT8_MAX).astype(np.int8)
    return q.reshape(x32.shape), s


def dequant_int8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float64 [..., K] = q * s of the value's 128-block."""
    return np.asarray(q, dtype=np.float64) * np.repeat(np.asarray(s, dtype=np.float64), BLOCK, axis=-1)
