"""Number formats: OCP FP8 E4M3 (decode table, round-to-nearest-even encode),
OCP FP4 E2M1 and its E8M0 block scales, bf16 and fp16 bit patterns.
TEST INFRASTRUCTURE ONLY (see package header).

[DG-FP8] describes E4M3 as 1 sign bit, 4 exponent bits and 3 mantissa bits
with a range of about +-448.  The +-448 range identifies the OCP "E4M3FN"
variant (exponent bias 7, no infinities, only S.1111.111 is NaN); the FNUZ
variant tops out at 240.  The decode below is that format's definition.
"""

from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3FN code (bias 7; exponent field 0 is subnormal; 0x7F/0xFF NaN).

    Pinned by: closed-form values (0x01 = 2^-9, 0x08 = 2^-6, 0x38 = 1, 0x7E = 448),
    strict monotonicity of 0x00..0x7E, and equality with torch.float8_e4m3fn.
    """
    code = int(code) & 0xFF
    s = code >> 7
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        v = m * 2.0 ** -9  # subnormal: m/8 * 2^(1-7)
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def e4m3_decode_table() -> np.ndarray:
    """float64[256]: value of every code (NaN for the two NaN codes)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(v) -> np.ndarray:
    """Round float64 values to the nearest E4M3FN code, ties to the even code.

    The format's rounding rule written out: a magnitude below the smallest
    normal 2^-6 is a multiple of the subnormal step 2^-9 (code = that multiple,
    rounded half to even; 8 steps is the smallest normal, code 0x08); otherwise
    a = (1 + f) * 2^E with E in [-6, 8], the 3-bit mantissa is f * 8 rounded half
    to even, and code = (E + 7) * 8 + mantissa (a carry into the exponent is the
    next binade, exactly as the code order continues).

    Requires |v| <= 448 (the quantiser guarantees it, so no saturation rule is
    needed).  The sign is carried even when the magnitude rounds to zero, so
    tiny negative inputs give 0x80.

    Pinned by: exhaustive comparison with torch's float8_e4m3fn cast over every
    finite bf16 with |x| <= 448, and encode(decode(c)) == c for all finite codes.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    a = np.abs(v)
    if (a > E4M3_MAX).any():
        raise ValueError("e4m3_encode: |v| > 448")
    sub = a < 2.0 ** -6
    code_sub = np.rint(a * 2.0 ** 9)                      # np.rint rounds half to even; exact scaling
    _, ex = np.frexp(np.where(sub, 1.0, a))               # a = m * 2^ex, m in [0.5, 1)
    E = ex - 1                                            # a = (1 + f) * 2^E
    frac = np.where(sub, 0.0, np.ldexp(a, -E) - 1.0)      # exact
    code_norm = (E + 7) * 8 + np.rint(frac * 8.0)
    code = np.where(sub, code_sub, code_norm).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 7)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 patterns -> float64 (exact: bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even), returned as uint16 patterns.

    Used to compare a bf16 output with the value an exact result rounds to.
    Rounds the float64 directly (no intermediate fp32), via the exact neighbour
    comparison.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    for i, val in enumerate(flat_x):
        flat_o[i] = _bf16_rne_scalar(float(val))
    return out


def f64_to_bf16_bits_normal(x) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even) as uint16 patterns, vectorised, for values that are zero or
    whose magnitude lies in bf16's normal range [2^-126, 2^128); raises otherwise.

    With x = m * 2^e (frexp, 0.5 <= |m| < 1), bf16 keeps 8 significant bits: the result is
    rint(m * 2^8) * 2^(e-8), where the scaling is exact and np.rint rounds half to even.

    Pinned by: equality with f64_to_bf16_bits (the neighbour-comparison rounding) on random values
    spanning many binades, on exact halfway cases and on the carry into the next binade.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.isnan(x).any() or ((a != 0) & (a < 2.0 ** -126)).any() or (a >= 2.0 ** 128).any():
        raise ValueError("f64_to_bf16_bits_normal: value outside the normal range of bf16")
    m, e = np.frexp(x)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)      # may carry to the next power of two: still exact
    if (np.abs(r) >= 2.0 ** 128).any():
        raise ValueError("f64_to_bf16_bits_normal: rounds past the bf16 range")
    bits = r.astype(np.float32).view(np.uint32)          # r has 8 significant bits: exact in fp32
    return (bits >> 16).astype(np.uint16)


def _bf16_rne_scalar(val: float) -> int:
    if math.isnan(val):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, val) < 0 else 0
    a = abs(val)
    if a == 0.0:
        return sign
    # candidates: truncation toward zero of a to bf16 and the next pattern up
    f32 = np.array([a], dtype=np.float64).astype(np.float32)  # may round; fix below
    bits = int(f32.view(np.uint32)[0]) >> 16
    # walk to the largest bf16 pattern whose value <= a
    def val_of(b):
        return float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])
    while bits > 0 and val_of(bits) > a:
        bits -= 1
    while val_of(bits + 1) <= a and bits + 1 < 0x7F80:
        bits += 1
    lo_v, hi_v = val_of(bits), val_of(bits + 1)
    if lo_v == a:
        return sign | bits
    d_lo, d_hi = a - lo_v, hi_v - a
    if d_hi < d_lo or (d_hi == d_lo and (bits & 1)):
        bits += 1
    return sign | bits


def fp16_bits_to_f64(bits) -> np.ndarray:
    """uint16 IEEE half patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------------------------- FP4 E2M1 --
# The pages name 4-bit floating-point weights (E2M1: 1 sign, 2 exponent, 1 mantissa bit) in the MXFP4 and
# NVFP4 block-scaled forms ([CuTeDSL] Blackwell quantisation schemes; [AsymGEMM] "API Reference", FP4).  The
# element format is OCP E2M1: exponent bias 1, exponent field 0 subnormal (0 and 0.5), no infinities or NaN,
# largest magnitude 6.
E2M1_MAX = 6.0


def e2m1_value(code: int) -> float:
    """Value of one E2M1 code (low 4 bits).

    Pinned by: the closed-form table 0, 0.5, 1, 1.5, 2, 3, 4, 6 (and negatives) and strict monotonicity.
    """
    code = int(code) & 0xF
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    v = m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -v if s else v


def e2m1_decode_table() -> np.ndarray:
    """float64[16]: value of every E2M1 code."""
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m1_encode(v) -> np.ndarray:
    """Round float64 values to the nearest E2M1 code, ties to the code with an even mantissa bit.

    The rule written out: magnitudes below 1 are multiples of the subnormal step 0.5 (rounded half to even:
    0.25 -> 0, 0.75 -> 1.0); otherwise a = (1 + f) * 2^E with E in {0, 1, 2} and the 1-bit mantissa f * 2
    rounded half to even, a carry moving to the next binade.  Requires |v| <= 6; the sign is kept for values
    that round to zero.

    Pinned by: comparison with a nearest-value search over the eight magnitudes (ties broken toward the
    even code) on a dense grid including every halfway point, and encode(decode(c)) == c.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e2m1_encode: NaN input")
    a = np.abs(v)
    if (a > E2M1_MAX).any():
        raise ValueError("e2m1_encode: |v| > 6")
    sub = a < 1.0
    code_sub = np.rint(a * 2.0)                            # 0, 1 or 2 (2 is the code of 1.0)
    _, ex = np.frexp(np.where(sub, 1.0, a))
    E = ex - 1                                             # a = (1 + f) * 2^E, E in 0..2
    frac = np.where(sub, 0.0, np.ldexp(a, -E) - 1.0)
    code_norm = (E + 1) * 2 + np.rint(frac * 2.0)
    code = np.where(sub, code_sub, code_norm).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def e8m0_value(byte) -> np.ndarray:
    """Value 2^(b - 127) of E8M0 scale bytes (255, the NaN encoding, is rejected)."""
    b = np.asarray(byte, dtype=np.int64)
    if (b == 255).any():
        raise ValueError("E8M0 255 is NaN")
    return np.ldexp(np.ones(b.shape), b - 127)
