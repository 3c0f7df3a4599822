"""Pins for the oracle's number formats (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import e4m3_decode_table, e4m3_encode, e4m3_value


def test_e4m3_closed_form_values():
    # values fixed by the E4M3FN definition (bias 7, 3 mantissa bits, +-448 range)
    assert e4m3_value(0x00) == 0.0
    assert e4m3_value(0x01) == 2.0 ** -9          # smallest subnormal
    assert e4m3_value(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert e4m3_value(0x08) == 2.0 ** -6          # smallest normal
    assert e4m3_value(0x38) == 1.0
    assert e4m3_value(0x3C) == 1.5
    assert e4m3_value(0x40) == 2.0
    assert e4m3_value(0x7E) == 448.0              # the page's +-448 range
    assert e4m3_value(0xFE) == -448.0
    assert math.copysign(1.0, e4m3_value(0x80)) == -1.0 and e4m3_value(0x80) == 0.0
    assert math.isnan(e4m3_value(0x7F)) and math.isnan(e4m3_value(0xFF))


def test_e4m3_table_invariants():
    tab = e4m3_decode_table()
    assert np.isnan(tab).sum() == 2
    pos = tab[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must be strictly increasing"
    assert np.array_equal(tab[0x80:0xFF], -tab[:0x7F])


def test_e4m3_table_matches_torch():
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = e4m3_decode_table()
    both_nan = np.isnan(t) & np.isnan(tab)
    assert np.array_equal(both_nan, np.isnan(t)) and np.array_equal(both_nan, np.isnan(tab))
    ok = both_nan | (t == tab)
    assert ok.all()


def _all_bf16_in_range():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    return bits[keep], vals[keep]


def test_e4m3_encode_exhaustive_vs_torch_cast():
    bits, vals = _all_bf16_in_range()
    ours = e4m3_encode(vals)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mism = np.nonzero(ours != ref)[0]
    assert mism.size == 0, f"{mism.size} mismatches, first value {vals[mism[0]]!r}"
    assert bits.size > 34000


def test_e4m3_encode_roundtrip_and_sign():
    tab = e4m3_decode_table()
    for c in range(256):
        if math.isnan(tab[c]):
            continue
        assert int(e4m3_encode(np.array([tab[c]]))[0]) == c
    assert int(e4m3_encode(np.array([-1e-4]))[0]) == 0x80
    assert int(e4m3_encode(np.array([2.0 ** -10]))[0]) == 0x00       # tie between 0 and 2^-9 -> even code 0
    assert int(e4m3_encode(np.array([3 * 2.0 ** -10]))[0]) == 0x02   # tie between 0x01 and 0x02 -> 0x02
    assert int(e4m3_encode(np.array([1.0625]))[0]) == 0x38           # tie 1 / 1.125 -> even (0x38)
    assert int(e4m3_encode(np.array([1.1875]))[0]) == 0x3A           # tie 1.125 / 1.25 -> even (0x3A)
    with pytest.raises(ValueError):
        e4m3_encode(np.array([449.0]))


def test_bf16_fp16_decode():
    assert oracle.bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert oracle.bf16_bits_to_f64(np.array([0xC000], np.uint16))[0] == -2.0
    assert oracle.fp16_bits_to_f64(np.array([0x3C00], np.uint16))[0] == 1.0
    assert oracle.fp16_bits_to_f64(np.array([0x0001], np.uint16))[0] == 2.0 ** -24
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -3.14159, 0.0, 1e-40])
    got = oracle.f64_to_bf16_bits(x)
    ref = torch.tensor(x, dtype=torch.float64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_vectorised_bf16_rounding_equals_the_neighbour_rounding():
    rng = np.random.default_rng(17)
    x = rng.standard_normal(4000) * 2.0 ** rng.integers(-100, 100, 4000)
    # exact halfway points between neighbours (ties to even) and the carry into the next binade
    base = oracle.bf16_bits_to_f64(np.arange(0x3F80, 0x3F80 + 300, dtype=np.uint16))
    half = (base[:-1] + base[1:]) / 2
    edge = np.array([2.0 - 2.0 ** -9, 2.0 - 2.0 ** -8 - 2.0 ** -10, -(1.0 + 2.0 ** -8), 0.0, -0.0, 3.0e38])
    for v in (x, half, -half, edge):
        assert np.array_equal(oracle.f64_to_bf16_bits_normal(v), oracle.f64_to_bf16_bits(v))
    with pytest.raises(ValueError):
        oracle.f64_to_bf16_bits_normal(np.array([1e-40]))
