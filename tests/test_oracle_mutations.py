"""Plant plausible mistakes in the oracle (CPU only) and check a pin catches each.

Each case patches one oracle function for the duration of the test and runs a
pin from the other test modules; the pin must fail.
"""

import numpy as np
import pytest

import oracle
import oracle.gemm as og
import oracle.routing as orr
import test_oracle_formats as tf
import test_oracle_gemm as tg
import test_oracle_routing as tr


def _expect_fail(fn):
    with pytest.raises(AssertionError):
        fn()


def test_mutation_wrong_exponent_bias_is_caught(monkeypatch):
    orig = tf.e4m3_value

    def biased(code):
        v = orig(code)
        return v * 2.0 if v == v else v  # bias 6 instead of 7

    monkeypatch.setattr(tf, "e4m3_value", biased)
    _expect_fail(tf.test_e4m3_closed_form_values)


def test_mutation_ties_away_from_zero_is_caught(monkeypatch):
    orig = tf.e4m3_encode

    def away(v):
        v = np.asarray(v, dtype=np.float64)
        # nudge ties up: round-half-away instead of half-even
        return orig(np.clip(v * (1 + 2.0 ** -40), -448.0, 448.0))

    monkeypatch.setattr(tf, "e4m3_encode", away)
    _expect_fail(tf.test_e4m3_encode_exhaustive_vs_torch_cast)


def test_mutation_reverse_order_within_expert_is_caught(monkeypatch):
    orig = orr.route

    def reversed_route(ids, E, layout="contiguous", align=128, max_m=0, rows_cap=None):
        r = orig(ids, E, layout, align, max_m, rows_cap)
        oi = r["output_index"].reshape(-1).copy()
        for e in range(E):
            sel = np.nonzero(np.asarray(ids).reshape(-1) == e)[0]
            oi[sel] = oi[sel][::-1]
        r["output_index"] = oi.reshape(r["output_index"].shape)
        return r

    monkeypatch.setattr(oracle, "route", reversed_route)
    _expect_fail(tr.test_worked_example_aligned_128)


def test_mutation_unaligned_segments_are_caught(monkeypatch):
    orig = orr.route
    monkeypatch.setattr(oracle, "route", lambda ids, E, layout="contiguous", align=128, max_m=0, rows_cap=None:
                        orig(ids, E, layout, 1 if layout == "contiguous" else align, max_m, rows_cap))
    _expect_fail(tr.test_worked_example_aligned_128)


def test_mutation_dropped_block_scale_is_caught(monkeypatch):
    orig = og.grouped_gemm_fp8

    def no_wscale(a_codes, sfa, w_codes, sfw, counts, seg_offsets, rows_out=None, experts=None):
        return orig(a_codes, sfa, w_codes, np.ones_like(sfw), counts, seg_offsets, rows_out, experts)

    monkeypatch.setattr(oracle, "grouped_gemm_fp8", no_wscale)
    _expect_fail(tg.test_fp8_gemm_exact_rational_brute_force)


def test_mutation_transposed_weight_is_caught(monkeypatch):
    def transposed(a_bits, w_q4, s16_bits, counts, seg_offsets, rows_out=None, experts=None):
        # reads the wrong nibble of each byte (high nibble as the even k)
        swapped = ((w_q4 >> 4) | ((w_q4 & 15) << 4)).astype(np.uint8)
        return og.grouped_gemm_int4(a_bits, swapped, s16_bits, counts, seg_offsets, rows_out, experts)

    monkeypatch.setattr(oracle, "grouped_gemm_int4", transposed)
    _expect_fail(tg.test_int4_gemm_integer_case_and_brute_force)


def test_mutation_combine_wrong_slot_weight_is_caught(monkeypatch):
    orig = oracle.combine
    monkeypatch.setattr(oracle, "combine", lambda y, oi, w: orig(y, oi, w[:, ::-1].copy()))
    _expect_fail(tg.test_combine_worked_example_and_brute_force)


def test_mutation_sigmoid_instead_of_silu_is_caught(monkeypatch):
    import test_oracle_activation as ta
    monkeypatch.setattr(oracle, "silu", lambda x: 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64))))
    _expect_fail(ta.test_silu_closed_forms)


def test_mutation_up_then_gate_is_caught(monkeypatch):
    import oracle.activation as oa
    import test_oracle_activation as ta
    orig = oa.swiglu

    def swapped(gu):
        gu = np.asarray(gu, np.float64)
        i = gu.shape[1] // 2
        return orig(np.concatenate([gu[:, i:], gu[:, :i]], axis=1))

    monkeypatch.setattr(oracle, "swiglu", swapped)
    _expect_fail(ta.test_swiglu_takes_gate_then_up)


def test_mutation_fma_rounded_twice_is_caught(monkeypatch):
    import importlib
    import test_oracle_combine as tc
    oc = importlib.import_module("oracle.combine")
    monkeypatch.setattr(oc, "_fma_f32", lambda w, y, acc: (w.astype(np.float32) * y.astype(np.float32) + acc)
                        .astype(np.float32))
    _expect_fail(tc.test_fma_step_is_the_exactly_rounded_fused_multiply_add)


def test_mutation_bf16_transposed_weight_is_caught(monkeypatch):
    orig = og.grouped_gemm_bf16

    def transposed(a_bits, w_bits, counts, seg_offsets, rows_out=None, experts=None):
        # weights read K-major from an [E, K, N] view of the same bytes
        E, N, K = w_bits.shape
        wt = np.ascontiguousarray(w_bits.reshape(E, K, N).transpose(0, 2, 1))
        return orig(a_bits, wt, counts, seg_offsets, rows_out, experts)

    monkeypatch.setattr(oracle, "grouped_gemm_bf16", transposed)
    _expect_fail(tg.test_bf16_gemm_exact_rational_brute_force)


def test_mutation_fp4_nibble_order_is_caught(monkeypatch):
    import oracle.gemm as og2
    import test_oracle_fp4 as tf4
    orig = og2.grouped_gemm_fp8_fp4

    def swapped(a, sa, w4, sw, counts, seg, rows_out=None, experts=None):
        return orig(a, sa, ((w4 >> 4) | ((w4 & 15) << 4)).astype(np.uint8), sw, counts, seg, rows_out, experts)

    monkeypatch.setattr(oracle, "grouped_gemm_fp8_fp4", swapped)
    _expect_fail(tf4.test_fp8_fp4_gemm_exact_rational_brute_force)


def test_mutation_fp4_ties_away_is_caught(monkeypatch):
    import test_oracle_fp4 as tf4
    orig = oracle.e2m1_encode
    monkeypatch.setattr(oracle, "e2m1_encode", lambda v: orig(np.clip(np.asarray(v, np.float64) * (1 + 1e-12), -6, 6)))
    _expect_fail(tf4.test_e2m1_encode_equals_nearest_search_on_a_dense_grid)
