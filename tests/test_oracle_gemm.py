"""Pins for the oracle's grouped GEMMs, combine and metrics (CPU only)."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import e4m3_value

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _rand_codes(rng, shape, pool=None):
    if pool is None:  # every finite code
        pool = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    return rng.choice(pool, size=shape).astype(np.uint8)


def _pow2(rng, shape, lo=-4, hi=4):
    return np.ldexp(np.ones(shape), rng.integers(lo, hi + 1, size=shape)).astype(np.float32)


def _fp8_problem(rng, E=2, K=256, N=128, counts=(3, 5), align=16):
    counts = np.array(counts, dtype=np.int32)
    starts = np.zeros(E + 1, dtype=np.int32)
    for e in range(E):
        starts[e + 1] = starts[e] + -(-counts[e] // align) * align
    rows = int(starts[E])
    a = _rand_codes(rng, (rows, K))
    sa = _pow2(rng, (rows, K // 128))
    w = _rand_codes(rng, (E, N, K))
    sw = _pow2(rng, (E, N // 128, K // 128))
    return a, sa, w, sw, counts, starts


def test_fp8_gemm_exact_rational_brute_force():
    rng = np.random.default_rng(0)
    a, sa, w, sw, counts, starts = _fp8_problem(rng)
    d = oracle.grouped_gemm_fp8(a, sa, w, sw, counts, starts)
    frac = {c: Fraction(e4m3_value(c)) for c in range(256) if c not in (0x7F, 0xFF)}
    cols = [0, 1, 63, 127]
    for e in range(2):
        for p in range(int(starts[e]), int(starts[e]) + int(counts[e])):
            for n in cols:
                exact = Fraction(0)
                for k in range(a.shape[1]):
                    exact += (frac[a[p, k]] * Fraction(float(sa[p, k // 128])) *
                              frac[w[e, n, k]] * Fraction(float(sw[e, n // 128, k // 128])))
                assert d[p, n] == float(exact)
    # rows outside the segments are NaN
    assert np.isnan(d[int(starts[0]) + int(counts[0]):int(starts[1])]).all()


def test_fp8_gemm_one_hot_closed_form():
    rng = np.random.default_rng(1)
    a, sa, w, sw, counts, starts = _fp8_problem(rng)
    a[:] = 0
    k0 = 77
    a[0, k0] = 0x40  # 2.0
    sa[0, :] = 1.0
    d = oracle.grouped_gemm_fp8(a, sa, w, sw, counts, starts)
    tab = oracle.e4m3_decode_table()
    ref = 2.0 * tab[w[0, :, k0]] * sw[0, np.arange(128) // 128, k0 // 128]
    assert np.array_equal(d[0], ref)


def test_fp8_gemm_small_integers_match_integer_matmul():
    rng = np.random.default_rng(2)
    # codes whose values are the integers -4..4
    ints = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}
    vals = np.arange(-4, 5)
    code_of = {v: (ints[abs(v)] | (0x80 if v < 0 else 0)) for v in vals}
    E, K, N = 2, 256, 128
    counts = np.array([4, 6], np.int32)
    starts = np.array([0, 16, 32], np.int32)
    ai = rng.integers(-4, 5, size=(32, K))
    wi = rng.integers(-4, 5, size=(E, N, K))
    a = np.vectorize(code_of.get)(ai).astype(np.uint8)
    w = np.vectorize(code_of.get)(wi).astype(np.uint8)
    d = oracle.grouped_gemm_fp8(a, np.ones((32, 2), np.float32), w, np.ones((E, 1, 2), np.float32), counts, starts)
    for e in range(E):
        s, c = starts[e], counts[e]
        assert np.array_equal(d[s:s + c], (ai[s:s + c] @ wi[e].T).astype(np.float64))


def test_fp8_gemm_scale_invariance():
    rng = np.random.default_rng(3)
    a, sa, w, sw, counts, starts = _fp8_problem(rng)
    d0 = oracle.grouped_gemm_fp8(a, sa, w, sw, counts, starts)
    d1 = oracle.grouped_gemm_fp8(a, sa * np.float32(8), w, sw / np.float32(8), counts, starts)
    d2 = oracle.grouped_gemm_fp8(a, sa * np.float32(4), w, sw, counts, starts)
    valid = ~np.isnan(d0)
    assert np.array_equal(d0[valid], d1[valid])
    assert np.array_equal(4 * d0[valid], d2[valid])


def test_fp8_gemm_equals_per_expert_single_gemms():
    rng = np.random.default_rng(4)
    a, sa, w, sw, counts, starts = _fp8_problem(rng, E=3, counts=(2, 0, 7))
    d = oracle.grouped_gemm_fp8(a, sa, w, sw, counts, starts)
    for e in range(3):
        s, c = int(starts[e]), int(counts[e])
        if c == 0:
            continue
        single = oracle.grouped_gemm_fp8(a[s:s + c], sa[s:s + c], w[e:e + 1], sw[e:e + 1],
                                         np.array([c]), np.array([0, c]))
        assert np.array_equal(d[s:s + c], single)


def test_int4_gemm_integer_case_and_brute_force():
    rng = np.random.default_rng(5)
    E, K, N = 2, 256, 16
    counts = np.array([3, 2], np.int32)
    starts = np.array([0, 4, 8], np.int32)
    ai = rng.integers(-3, 4, size=(8, K)).astype(np.float32)
    a_bits = torch.from_numpy(ai).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q = rng.integers(0, 16, size=(E, N, K)).astype(np.uint8)
    q4 = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    ones = np.full((E, N, K // 128), 0x3C00, np.uint16)
    d = oracle.grouped_gemm_int4(a_bits, q4, ones, counts, starts)
    for e in range(E):
        s, c = starts[e], counts[e]
        ref = ai[s:s + c].astype(np.int64) @ (q[e].astype(np.int64) - 8).T
        assert np.array_equal(d[s:s + c], ref.astype(np.float64))
    # brute force with fp16 scales
    s16 = rng.integers(0x2000, 0x4000, size=(E, N, K // 128)).astype(np.uint16)
    d2 = oracle.grouped_gemm_int4(a_bits, q4, s16, counts, starts)
    sv = s16.view(np.float16)
    for e in range(E):
        for p in range(int(starts[e]), int(starts[e]) + int(counts[e])):
            for n in (0, 7, 15):
                exact = sum(Fraction(float(ai[p, k])) * (int(q[e, n, k]) - 8) * Fraction(float(sv[e, n, k // 128]))
                            for k in range(K))
                assert d2[p, n] == float(exact)


def test_combine_worked_example_and_brute_force():
    with open(GOLDEN, encoding="utf-8") as f:
        g = json.load(f)
    ids = np.array(g["topk_ids"], np.int32)
    wts = np.array(g["topk_weights"], np.float64)
    r = oracle.route(ids, 4, "contiguous", align=128)
    rng = np.random.default_rng(6)
    y = rng.standard_normal((r["rows_cap"], 8))
    z = oracle.combine(y, r["output_index"], wts)
    (p0, w0), (p1, w1) = g["aligned128"]["z0_rows_and_weights"]
    assert z[0].tolist() == (w0 * y[p0] + w1 * y[p1]).tolist()
    ru = oracle.route(ids, 4, "contiguous", align=1)
    zu = oracle.combine(y, ru["output_index"], wts)
    (q0, v0), (q1, v1) = g["unaligned"]["z0_rows_and_weights"]
    assert zu[0].tolist() == (v0 * y[q0] + v1 * y[q1]).tolist()
    # exact rational brute force over all tokens with a dropped slot
    oi = r["output_index"].copy()
    oi[3, 1] = -1
    z2 = oracle.combine(y, oi, wts)
    for t in range(5):
        for n in range(8):
            exact = sum(Fraction(float(wts[t, s])) * Fraction(float(y[oi[t, s], n])) for s in range(2) if oi[t, s] >= 0)
            assert abs(z2[t, n] - float(exact)) <= 2 ** -50 * (abs(float(exact)) + 1)


def test_calc_diff_closed_forms():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(1000)
    assert oracle.calc_diff(x, x) == pytest.approx(0.0, abs=1e-15)
    assert oracle.calc_diff(x, -x) == pytest.approx(2.0)
    for c in (0.5, 0.999, 2.0):
        assert oracle.calc_diff(x, c * x) == pytest.approx((1 - c) ** 2 / (1 + c * c), rel=1e-9, abs=1e-15)
    assert oracle.calc_diff(np.zeros(4), np.zeros(4)) == 0.0
    assert oracle.elementwise_ok(x, x) and not oracle.elementwise_ok(x + 1.0, x)


def _bf16_problem(rng, E=2, K=64, N=16, counts=(3, 5), align=8, scale=1.0):
    counts = np.array(counts, dtype=np.int32)
    starts = np.zeros(E + 1, dtype=np.int32)
    for e in range(E):
        starts[e + 1] = starts[e] + -(-counts[e] // align) * align
    rows = int(starts[E])
    a = oracle.f32_to_bf16_bits((rng.standard_normal((rows, K)) * scale).astype(np.float32))
    w = oracle.f32_to_bf16_bits((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32))
    return a, w, counts, starts


def test_bf16_gemm_exact_rational_brute_force():
    rng = np.random.default_rng(10)
    a, w, counts, starts = _bf16_problem(rng)
    d = oracle.grouped_gemm_bf16(a, w, counts, starts)
    af, wf = oracle.bf16_bits_to_f64(a), oracle.bf16_bits_to_f64(w)
    for e in range(2):
        for p in range(int(starts[e]), int(starts[e]) + int(counts[e])):
            for n in (0, 5, 15):
                exact = sum(Fraction(float(af[p, k])) * Fraction(float(wf[e, n, k])) for k in range(a.shape[1]))
                assert d[p, n] == float(exact)
    assert np.isnan(d[int(starts[0]) + int(counts[0]):int(starts[1])]).all()


def test_bf16_gemm_integers_one_hot_and_per_expert():
    rng = np.random.default_rng(11)
    E, K, N = 3, 128, 32
    counts = np.array([4, 0, 6], np.int32)
    starts = np.array([0, 8, 8, 16], np.int32)
    ai = rng.integers(-8, 9, size=(16, K)).astype(np.float32)
    wi = rng.integers(-8, 9, size=(E, N, K)).astype(np.float32)
    a, w = oracle.f32_to_bf16_bits(ai), oracle.f32_to_bf16_bits(wi)
    d = oracle.grouped_gemm_bf16(a, w, counts, starts)
    for e in (0, 2):
        s, c = starts[e], counts[e]
        assert np.array_equal(d[s:s + c], (ai[s:s + c].astype(np.int64) @ wi[e].astype(np.int64).T).astype(np.float64))
        single = oracle.grouped_gemm_bf16(a[s:s + c], w[e:e + 1], np.array([c]), np.array([0, c]))
        assert np.array_equal(d[s:s + c], single)
    # one-hot row: a single 1.0 at k0 picks column k0 of the weights
    a1 = np.zeros((16, K), np.uint16)
    a1[0, 37] = 0x3F80
    d1 = oracle.grouped_gemm_bf16(a1, w, counts, starts)
    assert np.array_equal(d1[0], wi[0, :, 37].astype(np.float64))
