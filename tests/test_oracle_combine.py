"""Pins of the oracle's combine: the float64 sum and the fp32 fma-chain form (reading A13).

combine_fp32 is pinned by three things that do not share its arithmetic:
  * exact rational evaluation: every fma computed in fractions.Fraction and
    rounded to fp32 by the definition of round-to-nearest-even (significand
    scaled to an integer, ties to the even integer), then rounded to bf16 by
    the same definition;
  * plain float32 arithmetic (numpy) where every product w*y is exact in fp32
    (weights with at most 16 significant bits), so fma == add of the product;
  * constructed cases where the float64 sum lands exactly halfway between two
    fp32 values but the exact sum does not (the one branch where a plain
    float64 -> fp32 rounding would be wrong).
"""

import importlib
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _rn_to_precision(q: Fraction, mant_bits: int, min_exp: int) -> Fraction:
    """Round a rational to the nearest value with `mant_bits` significant bits (ties to even), with
    subnormal spacing 2^(min_exp - mant_bits + 1) below 2^min_exp."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^e <= a < 2^(e+2); fix below
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, min_exp)
    ulp = Fraction(2) ** (e - mant_bits + 1)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * ulp
    return r if q > 0 else -r


def _rn_f32(q):
    return _rn_to_precision(q, 24, -126)


def _bf16_bits_of(q: Fraction) -> int:
    v = _rn_to_precision(q, 8, -126)
    f = np.float32(float(v))  # exact: v has 8 significant bits
    return int(np.array([f], np.float32).view(np.uint32)[0]) >> 16


def _brute(y_bits, oi, w):
    rows, N = y_bits.shape
    yv = (y_bits.astype(np.uint32) << 16).view(np.float32)
    T, k = oi.shape
    out = np.zeros((T, N), np.uint16)
    for t in range(T):
        for n in range(N):
            acc = Fraction(0)
            for r in range(k):
                p = int(oi[t, r])
                if p < 0 or p >= rows:
                    continue
                acc = _rn_f32(Fraction(float(w[t, r])) * Fraction(float(yv[p, n])) + acc)
            out[t, n] = _bf16_bits_of(acc)
    return out


def _bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return oracle.f32_to_bf16_bits(x)


@pytest.mark.parametrize("seed", range(4))
def test_combine_fp32_equals_exact_rational_fma_chain(seed):
    rng = np.random.default_rng(seed)
    rows, T, k, N = 12, 5, 6, 7
    y = _bf16(rng, (rows, N), scale=10.0 ** rng.integers(-3, 4))
    oi = rng.integers(-1, rows, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w[0] = -w[0]
    assert np.array_equal(oracle.combine_fp32(y, oi, w), _brute(y, oi, w))


def test_combine_fp32_equals_float32_arithmetic_when_products_are_exact():
    rng = np.random.default_rng(11)
    rows, T, k, N = 300, 200, 8, 64
    y = _bf16(rng, (rows, N))
    oi = rng.integers(-1, rows, size=(T, k)).astype(np.int32)
    w = (np.round(rng.random((T, k)) * 2 ** 16) / 2 ** 16).astype(np.float32)  # <= 16 significant bits
    yv = (y.astype(np.uint32) << 16).view(np.float32)
    acc = np.zeros((T, N), np.float32)
    for r in range(k):
        for t in range(T):
            p = oi[t, r]
            if p >= 0:
                acc[t] = acc[t] + w[t, r] * yv[p]   # the product is exact, so this is the fma
    assert np.array_equal(oracle.combine_fp32(y, oi, w), oracle.f32_to_bf16_bits(acc))


def _halfway_cases():
    """(acc, w, y) with acc + w*y off an fp32 halfway point by less than half a float64 ulp, both signs."""
    cases = []
    acc = np.float32(2.0 ** 24)            # fp32 spacing 2 at and above 2^24
    for ym in range(129, 256, 2):          # y = ym / 128, an 8-bit significand
        y = np.float32(ym / 128.0)
        for j in range(3):
            target = Fraction(2 * j + 1)   # (j + 1/2) * spacing
            w = np.float32(float(target / Fraction(ym, 128)))
            d = Fraction(float(w)) * Fraction(ym, 128) - target
            s = float(Fraction(float(acc)) + Fraction(float(w)) * Fraction(ym, 128))
            if d != 0 and s == float(2 ** 24 + 2 * j + 1):
                cases.append((acc, w, y, d > 0))
    return cases


def test_combine_fp32_halfway_sums_round_by_the_exact_value():
    cases = _halfway_cases()
    signs = {c[3] for c in cases}
    assert len(cases) >= 4 and signs == {True, False}, "the construction must hit both directions"
    for acc, w, y, _ in cases:
        # slot 0 puts acc in the accumulator exactly (weight 1, y = acc needs acc to be bf16: 2^24 is)
        yb = oracle.f32_to_bf16_bits(np.array([[acc], [y]], np.float32))
        oi = np.array([[0, 1]], np.int32)
        wt = np.array([[1.0, w]], np.float32)
        got = oracle.combine_fp32(yb, oi, wt)
        assert np.array_equal(got, _brute(yb, oi, wt))
        # and the fp32 accumulator itself (before the bf16 rounding) is the exact rational rounding
        f = importlib.import_module("oracle.combine")._fma_f32(np.array([w]), np.array([y]), np.array([acc], np.float32))[0]
        want = _rn_f32(Fraction(float(acc)) + Fraction(float(w)) * Fraction(float(y)))
        assert Fraction(float(f)) == want


def test_combine_fp32_within_bound_of_float64_combine():
    rng = np.random.default_rng(3)
    rows, T, k, N = 400, 100, 8, 96
    y = _bf16(rng, (rows, N))
    oi = rng.integers(-1, rows, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    z = oracle.bf16_bits_to_f64(oracle.combine_fp32(y, oi, w))
    yf = oracle.bf16_bits_to_f64(y)
    ref = oracle.combine(yf, oi, w.astype(np.float64))
    mag = oracle.combine(np.abs(yf), oi, np.abs(w.astype(np.float64)))
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.maximum(np.abs(ref), np.abs(z)), 2.0 ** -126))) - 7)
    assert (np.abs(z - ref) <= 0.5 * ulp + (k + 1) * 2.0 ** -24 * mag).all()


def test_combine_fp32_worked_example_and_empty_slots():
    g = json.load(open(GOLDEN, encoding="utf-8"))
    ids = np.array(g["topk_ids"], np.int32)
    w = np.array(g["topk_weights"], np.float32)
    r = oracle.route(ids, 4, "contiguous", align=128)
    rng = np.random.default_rng(0)
    y = _bf16(rng, (r["rows_cap"], 16))
    z = oracle.combine_fp32(y, r["output_index"], w)
    assert np.array_equal(z[:2], _brute(y, r["output_index"][:2], w[:2]))
    # z_0 = 0.70 * y[0] + 0.30 * y[256] (the page's z_0), as an fp32 fma chain
    assert list(r["output_index"][0]) == [0, 256]
    # all slots dropped: +0
    z2 = oracle.combine_fp32(y, np.full((3, 2), -1, np.int32), np.ones((3, 2), np.float32))
    assert (z2 == 0).all()


def test_fma_step_is_the_exactly_rounded_fused_multiply_add():
    """Each step rounds once: RN_f32(w*y + acc) for random fp32 w, acc and bf16 y over wide exponent ranges."""
    rng = np.random.default_rng(21)
    n = 3000
    w = (rng.standard_normal(n) * 2.0 ** rng.integers(-20, 20, n)).astype(np.float32)
    y = (oracle.f32_to_bf16_bits((rng.standard_normal(n) * 2.0 ** rng.integers(-20, 20, n)).astype(np.float32))
         .astype(np.uint32) << 16).view(np.float32)
    acc = (rng.standard_normal(n) * 2.0 ** rng.integers(-30, 30, n)).astype(np.float32)
    got = importlib.import_module("oracle.combine")._fma_f32(w, y, acc)
    for i in range(n):
        want = _rn_f32(Fraction(float(w[i])) * Fraction(float(y[i])) + Fraction(float(acc[i])))
        assert Fraction(float(got[i])) == want, i
