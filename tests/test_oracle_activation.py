"""Pins of the oracle's SwiGLU and its requantisation (values the mathematics fixes)."""

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle


def test_silu_closed_forms():
    ln3 = math.log(3.0)
    s = oracle.silu(np.array([0.0, ln3, -ln3, 40.0]))
    assert s[0] == 0.0
    assert s[1] == pytest.approx(0.75 * ln3, rel=2e-16, abs=0)
    assert s[2] == pytest.approx(-0.25 * ln3, rel=4e-16, abs=0)
    assert s[3] == 40.0  # sigmoid(40) rounds to 1 in float64
    big = oracle.silu(np.array([-800.0, 800.0]))
    assert big[0] == 0.0 and not np.isnan(big).any() and big[1] == 800.0


def test_silu_odd_part_identity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000) * 6
    assert np.allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=1e-15, atol=1e-15)


def test_silu_against_40_digit_decimal():
    getcontext().prec = 40
    rng = np.random.default_rng(2)
    for x in rng.standard_normal(300) * 8:
        d = Decimal(float(x))
        want = d / (1 + (-d).exp())
        got = oracle.silu(np.array([x]))[0]
        assert abs(Decimal(float(got)) - want) <= abs(want) * Decimal(2) ** -51 + Decimal(10) ** -300


def test_swiglu_takes_gate_then_up():
    g = np.array([[0.0, 30.0, -1.5, 2.0]])      # gate columns 0..1, up columns 2..3 (I = 2)
    h = oracle.swiglu(g)
    assert h.shape == (1, 2)
    assert h[0, 0] == 0.0                          # silu(0) * up = 0
    assert h[0, 1] == pytest.approx(2.0 * 30.0, rel=1e-12)  # silu(30) ~ 30
    # swapping the halves changes the result (the order matters and is the reading taken)
    assert not np.allclose(oracle.swiglu(g[:, [2, 3, 0, 1]]), h)


def test_quant_act_values_equals_quant_act_on_bf16_inputs():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((16, 384)) * 10.0 ** rng.integers(-4, 4, (16, 1))).astype(np.float32)
    bits = oracle.f32_to_bf16_bits(x)
    c1, s1 = oracle.quant_act(bits)
    c2, s2 = oracle.quant_act_values(oracle.bf16_bits_to_f64(bits))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_swiglu_quant_bounds_and_minimal_scales():
    rng = np.random.default_rng(4)
    gu = rng.standard_normal((40, 512)) * 3
    codes, sf = oracle.swiglu_quant(gu)
    h = oracle.swiglu(gu)
    assert codes.shape == (40, 256) and sf.shape == (40, 2)
    deq = oracle.dequant_act(codes, sf)
    s = np.repeat(sf.astype(np.float64), 128, axis=1)
    # E4M3 keeps 3 mantissa bits: error <= 2^-4 relative, or half the subnormal step 2^-10 * scale
    assert (np.abs(deq - h) <= np.maximum(2.0 ** -4 * np.abs(h), 2.0 ** -10 * s) + 1e-300).all()
    amax = np.abs(h.reshape(40, 2, 128)).max(axis=2)
    assert (amax <= 448.0 * sf).all() and (amax > 224.0 * sf).all()
