"""Pins of the oracle's FP4 (E2M1 + E8M0 block scales) format, quantiser and FP8 x FP4 grouped GEMM."""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def test_e2m1_closed_form_table():
    tab = oracle.e2m1_decode_table()
    assert tab[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert (tab[8:] == -tab[:8]).all() and math.copysign(1.0, tab[8]) < 0
    assert (np.diff(tab[:8]) > 0).all()


def _nearest_even(a):
    """Nearest of the eight E2M1 magnitudes by search; ties to the code with an even low bit."""
    mags = oracle.e2m1_decode_table()[:8]
    d = np.abs(mags - a)
    best = np.nonzero(d == d.min())[0]
    return int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])


def test_e2m1_encode_equals_nearest_search_on_a_dense_grid():
    grid = np.concatenate([np.arange(0, 6.0 + 1e-9, 1.0 / 64), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]])
    for a in grid:
        for sgn in (1.0, -1.0):
            c = int(oracle.e2m1_encode(np.array([sgn * a]))[0])
            assert c & 7 == _nearest_even(a), a
            assert (c >> 3) == (1 if sgn < 0 else 0)
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(oracle.e2m1_encode(oracle.e2m1_decode_table()), codes)


def test_fp4_scale_rule_minimal_and_bounded():
    rng = np.random.default_rng(1)
    for amax in np.concatenate([rng.random(500) * 10.0 ** rng.integers(-20, 20, 500), [6.0, 3.0, 6.0000001, 1e-40]]):
        e = oracle.pow2_exponent_e2m1(amax)
        assert amax <= 6.0 * 2.0 ** e and (amax > 3.0 * 2.0 ** e or e == -127)  # -127: the E8M0 clamp
    assert oracle.pow2_exponent_e2m1(0.0) == 0


def test_quant_weight_fp4_bounds_and_rescale_invariance():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((2, 16, 256)) * 0.02).astype(np.float32)
    bits = oracle.f32_to_bf16_bits(w)
    w4, sw = oracle.quant_weight_fp4(bits)
    assert w4.shape == (2, 16, 128) and sw.shape == (2, 16, 8)
    x = oracle.bf16_bits_to_f64(bits)
    deq = oracle.dequant_weight_fp4(w4, sw)
    s = np.repeat(oracle.e8m0_value(sw), 32, axis=-1)
    # E2M1 keeps one mantissa bit: error <= a quarter of the value's binade, or 0.25 * scale below 1 * scale
    assert (np.abs(deq - x) <= np.maximum(0.25 * np.abs(x), 0.25 * s) + 1e-300).all()
    amax = np.abs(x.reshape(2, 16, 8, 32)).max(axis=3)
    assert (amax <= 6 * oracle.e8m0_value(sw)).all() and (amax > 3 * oracle.e8m0_value(sw)).all()
    # 2^j * w: same codes, scale bytes + j (every value stays a normal bf16)
    w4b, swb = oracle.quant_weight_fp4(oracle.f32_to_bf16_bits(w * np.float32(2.0 ** 5)))
    assert np.array_equal(w4b, w4) and np.array_equal(swb.astype(int), sw.astype(int) + 5)


def _problem(rng, E=2, K=256, N=16, counts=(3, 5), align=8):
    counts = np.array(counts, dtype=np.int32)
    starts = np.zeros(E + 1, dtype=np.int32)
    for e in range(E):
        starts[e + 1] = starts[e] + -(-counts[e] // align) * align
    rows = int(starts[E])
    pool = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    a = rng.choice(pool, size=(rows, K)).astype(np.uint8)
    sa = np.ldexp(np.ones((rows, K // 128)), rng.integers(-3, 4, (rows, K // 128))).astype(np.float32)
    w4 = rng.integers(0, 256, (E, N, K // 2)).astype(np.uint8)
    sw = rng.integers(120, 135, (E, N, K // 32)).astype(np.uint8)
    return a, sa, w4, sw, counts, starts


def test_fp8_fp4_gemm_exact_rational_brute_force():
    rng = np.random.default_rng(3)
    a, sa, w4, sw, counts, starts = _problem(rng)
    d = oracle.grouped_gemm_fp8_fp4(a, sa, w4, sw, counts, starts)
    f8 = {c: Fraction(oracle.e4m3_value(c)) for c in range(256) if c not in (0x7F, 0xFF)}
    f4 = [Fraction(oracle.e2m1_value(c)) for c in range(16)]
    for e in range(2):
        for p in range(int(starts[e]), int(starts[e]) + int(counts[e])):
            for n in (0, 9, 15):
                exact = Fraction(0)
                for k in range(a.shape[1]):
                    q = (int(w4[e, n, k // 2]) >> (4 * (k % 2))) & 15
                    exact += (f8[a[p, k]] * Fraction(float(sa[p, k // 128])) * f4[q] *
                              Fraction(2) ** (int(sw[e, n, k // 32]) - 127))
                assert d[p, n] == float(exact)
    assert np.isnan(d[int(starts[0]) + int(counts[0]):int(starts[1])]).all()


def test_fp8_fp4_gemm_integers_one_hot_scales_and_per_expert():
    rng = np.random.default_rng(4)
    E, K, N = 3, 256, 32
    counts = np.array([4, 0, 6], np.int32)
    starts = np.array([0, 8, 8, 16], np.int32)
    # activations: codes of -4..4; weights: E2M1 codes of -6..6 with all scales 1
    ints8 = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}
    ai = rng.integers(-4, 5, (16, K))
    a = np.vectorize(lambda v: ints8[abs(v)] | (0x80 if v < 0 else 0))(ai).astype(np.uint8)
    wv = rng.choice([-6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6], size=(E, N, K))
    q = oracle.e2m1_encode(wv.astype(np.float64))
    w4 = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    one = np.full((E, N, K // 32), 127, np.uint8)
    d = oracle.grouped_gemm_fp8_fp4(a, np.ones((16, 2), np.float32), w4, one, counts, starts)
    for e in (0, 2):
        s, c = starts[e], counts[e]
        assert np.array_equal(d[s:s + c], (ai[s:s + c] @ wv[e].T).astype(np.float64))
        single = oracle.grouped_gemm_fp8_fp4(a[s:s + c], np.ones((c, 2), np.float32), w4[e:e + 1], one[e:e + 1],
                                             np.array([c]), np.array([0, c]))
        assert np.array_equal(d[s:s + c], single)
    # one-hot activation row picks weight column k0 times its own block scale
    sw = rng.integers(120, 135, (E, N, K // 32)).astype(np.uint8)
    a1 = np.zeros((16, K), np.uint8)
    a1[0, 77] = 0x40  # 2.0
    d1 = oracle.grouped_gemm_fp8_fp4(a1, np.ones((16, 2), np.float32), w4, sw, counts, starts)
    assert np.array_equal(d1[0], 2.0 * wv[0, :, 77] * oracle.e8m0_value(sw[0, :, 77 // 32]))
    # scale invariance: sa * 2^j with weight scales - j leaves D unchanged
    d2 = oracle.grouped_gemm_fp8_fp4(a, np.full((16, 2), 8.0, np.float32), w4, (sw - 3).astype(np.uint8), counts,
                                     starts)
    d3 = oracle.grouped_gemm_fp8_fp4(a, np.ones((16, 2), np.float32), w4, sw, counts, starts)
    ok = ~np.isnan(d3)
    assert np.array_equal(d2[ok], d3[ok])
