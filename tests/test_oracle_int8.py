"""Pins of the INT8 (1, 1, 128) oracle ([AsymGEMM] "API Reference", INT8 asymmetric GEMM).

quant_int8 is checked against an exact rational evaluation of its defining steps (the fp32 roundings written
out from the definition of round-to-nearest-even) and against properties the rule must have; the grouped GEMM
against exact rational sums, integer matmuls and the factoring of the row and channel scales."""

from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rn(q: Fraction, mant_bits: int = 24, min_exp: int = -126) -> Fraction:
    """Round a rational to the nearest value with mant_bits significant bits (ties to even), subnormal spacing
    2^(min_exp - mant_bits + 1) below 2^min_exp (fp32 by default)."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
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


def _rint(q: Fraction) -> int:
    """Nearest integer, ties to even."""
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def _bf16(x):
    return oracle.f32_to_bf16_bits(np.asarray(x, np.float32))


def _blocks(rng):
    """bf16 rows of 128-blocks: random magnitudes over a wide range, tiny values, an all-zero block, a block with
    one nonzero value, and blocks whose values are ties of x / s (multiples of s / 2)."""
    rows = [rng.standard_normal(256) * 10.0 ** rng.integers(-6, 6), rng.standard_normal(256) * 1e-38,
            np.concatenate([np.zeros(128), np.eye(1, 128, 37)[0] * -3.5])]
    # ties: amax = 127 * 2^-3, values (n + 1/2) * 2^-3 (s = 2^-3 exactly)
    t = (np.arange(128) - 64 + 0.5) * 0.125
    t[5] = 127 * 0.125
    rows.append(np.concatenate([t, -t]))
    return _bf16(np.stack(rows))


def test_quant_int8_equals_exact_rational_steps():
    rng = np.random.default_rng(1)
    for _ in range(4):
        x_bits = _blocks(rng)
        q, s = oracle.quant_int8(x_bits)
        xv = oracle.bf16_bits_to_f64(x_bits)
        for r in range(xv.shape[0]):
            for b in range(xv.shape[1] // 128):
                blk = [Fraction(float(v)) for v in xv[r, 128 * b:128 * b + 128]]
                amax = max(abs(v) for v in blk)
                se = _rn(amax / 127) if amax > 0 else Fraction(1)
                assert Fraction(float(s[r, b])) == se, (r, b)
                for i, v in enumerate(blk):
                    qe = max(-127, min(127, _rint(_rn(v / se))))
                    assert int(q[r, 128 * b + i]) == qe, (r, b, i)


def test_quant_int8_properties():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 512)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    x_bits = _bf16(x)
    q, s = oracle.quant_int8(x_bits)
    xv = oracle.bf16_bits_to_f64(x_bits)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert (np.abs(q.astype(int)) <= 127).all()
    blk = xv.reshape(64, 4, 128)
    qb = q.reshape(64, 4, 128).astype(int)
    i = np.abs(blk).argmax(axis=2)
    assert (np.abs(np.take_along_axis(qb, i[..., None], 2)) == 127).all()  # the block's largest magnitude
    # half a step, plus the fp32 rounding of x / s (at most 127 * 2^-24 of a step) that can move a value
    # across a half-step boundary
    err = np.abs(xv - oracle.dequant_int8(q, s))
    assert (err <= np.repeat(s.astype(np.float64), 128, axis=1) * (0.5 + 127 * 2.0 ** -24)).all()
    qn, sn = oracle.quant_int8(_bf16(-oracle.bf16_bits_to_f64(x_bits)))  # sign symmetry
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    qj, sj = oracle.quant_int8(_bf16(xv * 2.0 ** 7))  # 2^j x: the same codes, scales times 2^j
    ok = np.isfinite(xv * 2.0 ** 7).all()
    assert ok and np.array_equal(qj, q) and np.array_equal(sj, s * np.float32(2.0 ** 7))
    qz, sz = oracle.quant_int8(np.zeros((2, 128), np.uint16))  # amax 0: scale 1, zero codes
    assert (qz == 0).all() and (sz == 1.0).all()


def _problem(rng, E=3, K=256, N=12, counts=(3, 0, 5), align=8, pow2=False):
    counts = np.array(counts, np.int32)
    starts = np.zeros(E + 1, np.int32)
    for e in range(E):
        starts[e + 1] = starts[e] + -(-counts[e] // align) * align
    rows = int(starts[E])
    a = rng.integers(-127, 128, (rows, K)).astype(np.int8)
    w = rng.integers(-127, 128, (E, N, K)).astype(np.int8)
    if pow2:
        sa = np.ldexp(1.0, rng.integers(-8, 3, (rows, K // 128))).astype(np.float32)
        sw = np.ldexp(1.0, rng.integers(-9, 1, (E, N, K // 128))).astype(np.float32)
    else:
        sa = rng.uniform(1e-3, 1.0, (rows, K // 128)).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-2, (E, N, K // 128)).astype(np.float32)
    return a, sa, w, sw, counts, starts


@pytest.mark.parametrize("pow2", [True, False])
def test_int8_gemm_exact_rational_brute_force(pow2):
    rng = np.random.default_rng(5)
    a, sa, w, sw, counts, starts = _problem(rng, pow2=pow2)
    d = oracle.grouped_gemm_int8(a, sa, w, sw, counts, starts)
    for e in (0, 2):
        for p in range(int(starts[e]), int(starts[e]) + int(counts[e])):
            for n in (0, 7, 11):
                exact = sum(Fraction(int(a[p, k]) * int(w[e, n, k])) * Fraction(float(sa[p, k // 128])) *
                            Fraction(float(sw[e, n, k // 128])) for k in range(a.shape[1]))
                if pow2:  # every product and partial sum exact in float64
                    assert d[p, n] == float(exact)
                else:
                    mag = sum(abs(int(a[p, k]) * int(w[e, n, k])) * float(sa[p, k // 128]) *
                              float(sw[e, n, k // 128]) for k in range(a.shape[1]))
                    assert abs(d[p, n] - float(exact)) <= 1e-14 * mag
    assert np.isnan(d[int(starts[0]) + int(counts[0]):int(starts[1])]).all()  # padding rows
    # a mistake in the scale indexing (the channel's scale of the wrong K block) is caught
    bad = sw[:, :, ::-1].copy()
    db = oracle.grouped_gemm_int8(a, sa, w, bad, counts, starts)
    assert not np.allclose(db[:3], d[:3])


def test_int8_gemm_integers_scale_factoring_and_per_expert():
    rng = np.random.default_rng(6)
    a, _, w, _, counts, starts = _problem(rng, E=3, K=384, N=16, counts=(5, 2, 0))
    rows = a.shape[0]
    one_a, one_w = np.ones((rows, 3), np.float32), np.ones((3, 16, 3), np.float32)
    d = oracle.grouped_gemm_int8(a, one_a, w, one_w, counts, starts)
    for e in (0, 1):
        s0, c = int(starts[e]), int(counts[e])
        assert np.array_equal(d[s0:s0 + c], (a[s0:s0 + c].astype(np.int64) @ w[e].T.astype(np.int64)).astype(float))
        single = oracle.grouped_gemm_int8(a[s0:s0 + c], one_a[s0:s0 + c], w[e:e + 1], one_w[e:e + 1],
                                          np.array([c]), np.array([0, c]))
        assert np.array_equal(d[s0:s0 + c], single)
    # a per-row scale constant over K scales that row; a per-channel one scales that column (powers of two: exact)
    sa = one_a.copy()
    sa[1] = 4.0
    sw = one_w.copy()
    sw[0, 3] = 0.5
    d2 = oracle.grouped_gemm_int8(a, sa, w, sw, counts, starts)
    expect = d.copy()
    expect[1] *= 4.0
    expect[starts[0]:starts[0] + counts[0], 3] *= 0.5
    ok = ~np.isnan(d)
    assert np.array_equal(d2[ok], expect[ok])


def test_int8_pins_catch_planted_mistakes(monkeypatch):
    """Rounding ties away from zero, or a scale of amax / 128, make the exact-steps pin fail."""
    import oracle.quant as Q
    real_rint = np.rint
    monkeypatch.setattr(Q.np, "rint", lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5))
    with pytest.raises(AssertionError):
        test_quant_int8_equals_exact_rational_steps()
    monkeypatch.setattr(Q.np, "rint", real_rint)
    monkeypatch.setattr(Q, "INT8_MAX", 128)
    with pytest.raises(AssertionError):
        test_quant_int8_equals_exact_rational_steps()
