"""Pins for the oracle's FP8 and INT4 quantisers (CPU only)."""

import math
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle.quant import pow2_exponent


def _bf16(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_pow2_exponent_minimality_random():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.lognormal(0, 6, 3000), [448.0, 448.0 * 2 ** 5, 448.0 * 2 ** -7, 447.9, 448.1,
                                                        1.0, 0.875 * 2 ** 9, 1e-30, 3e30]])
    for a in vals:
        e = pow2_exponent(a)
        if -126 < e < 127:
            assert a <= math.ldexp(448.0, e)
            assert a > math.ldexp(448.0, e - 1)
    assert pow2_exponent(0.0) == 0
    assert pow2_exponent(448.0) == 0
    assert pow2_exponent(449.0) == 1
    assert pow2_exponent(224.0) == -1
    assert pow2_exponent(1e-45) == -126  # clamp
    assert pow2_exponent(3e38) == 120  # 3e38/448 is just below 2^120


def test_pow2_exponent_equals_ceil_to_pow2_every_positive_bf16():
    # alternative definition: exponent of the power of two obtained by rounding
    # fp32(amax / 448) up to a power of two (the article's ceil_to_ue8m0 style)
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)  # positive finite bf16
    vals = oracle.bf16_bits_to_f64(bits)
    ratio = (vals.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    mant, ex = np.frexp(ratio.astype(np.float64))       # ratio = mant * 2^ex, mant in [0.5, 1)
    ceil_e = np.where(mant == 0.5, ex - 1, ex)
    ours = oracle.pow2_exponents(vals)
    ceil_e = np.clip(ceil_e, -126, 127)
    assert np.array_equal(ours, ceil_e)


def _is_pow2_f32(s):
    b = np.asarray(s, dtype=np.float32).view(np.uint32)
    return ((b & np.uint32(0x807FFFFF)) == 0) & (b != 0)


def test_quant_act_scales_are_pow2_and_bound_amax():
    torch.manual_seed(0)
    x = (torch.randn(7, 384) * torch.tensor([1e-3, 1.0, 300.0]).repeat_interleave(128)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    codes, sf = oracle.quant_act(bits)
    assert codes.shape == (7, 384) and sf.shape == (7, 3) and sf.dtype == np.float32
    assert _is_pow2_f32(sf).all()
    xf = oracle.bf16_bits_to_f64(bits).reshape(7, 3, 128)
    amax = np.abs(xf).max(axis=2)
    assert (amax <= 448.0 * sf).all() and (amax > 224.0 * sf).all()


def test_quant_act_rescale_invariance():
    torch.manual_seed(1)
    x = torch.randn(5, 256).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    c0, s0 = oracle.quant_act(bits)
    for j in (-5, -1, 1, 7):
        xj = (x.float() * 2.0 ** j).to(torch.bfloat16)  # exact: power-of-two rescale of bf16
        cj, sj = oracle.quant_act(xj.view(torch.int16).numpy().view(np.uint16))
        assert np.array_equal(c0, cj)
        assert np.array_equal(s0 * np.float32(2.0 ** j), sj)


def test_quant_act_error_bound_and_zero_block():
    torch.manual_seed(2)
    x = torch.randn(3, 256).to(torch.bfloat16)
    x[1, 128:] = 0
    bits = x.view(torch.int16).numpy().view(np.uint16)
    codes, sf = oracle.quant_act(bits)
    assert sf[1, 1] == 1.0 and (codes[1, 128:] == 0).all()
    deq = oracle.dequant_act(codes, sf)
    xf = oracle.bf16_bits_to_f64(bits)
    s = np.repeat(sf.astype(np.float64), 128, axis=1)
    # E4M3: relative half-ulp 2^-4 for normals, absolute half-ulp 2^-10 (times the scale) for subnormals
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, s * 2.0 ** -10)
    assert (np.abs(deq - xf) <= bound + 1e-300).all()


def test_quant_weight_fp8_blocks():
    torch.manual_seed(3)
    w = (torch.randn(2, 256, 256) * 0.02).to(torch.bfloat16)
    w[1, 128:, :128] *= 64
    bits = w.view(torch.int16).numpy().view(np.uint16)
    codes, sfw = oracle.quant_weight_fp8(bits)
    assert codes.shape == (2, 256, 256) and sfw.shape == (2, 2, 2)
    assert _is_pow2_f32(sfw).all()
    wf = oracle.bf16_bits_to_f64(bits)
    for e in range(2):
        for nb in range(2):
            for kb in range(2):
                blk = wf[e, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
                a = np.abs(blk).max()
                assert a <= 448 * sfw[e, nb, kb] and a > 224 * sfw[e, nb, kb]
    # a block's codes equal the 1x128 activation quantiser applied with the same scale:
    # rows of one 128x128 block quantised as activations whose amax equals the block amax
    e, nb, kb = 1, 1, 0
    blk_bits = bits[e, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
    deq = oracle.dequant_weight_fp8(codes, sfw)[e, nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
    assert np.max(np.abs(deq - oracle.bf16_bits_to_f64(blk_bits))) <= 448 * sfw[e, nb, kb] * 2.0 ** -4


def test_int4_nibble_table_exhaustive():
    b = np.arange(256, dtype=np.uint8)
    q = oracle.unpack_int4(b[None, :])[0]
    assert np.array_equal(q[0::2], b & 15) and np.array_equal(q[1::2], b >> 4)
    # dequant of every code with unit scale is q - 8
    q4 = np.array([[[(c & 15) | ((c & 15) << 4) for c in range(16)] * 4]], dtype=np.uint8)  # K = 128
    s = np.array([[[0x3C00]]], dtype=np.uint16)  # fp16 1.0
    d = oracle.dequant_weight_int4(q4, s)[0, 0]
    assert np.array_equal(d[0::2], np.arange(16, dtype=np.float64).repeat(1)[np.arange(64) % 16] - 8)


def test_quant_weight_int4_properties():
    torch.manual_seed(4)
    w = (torch.randn(2, 8, 256) * 0.02).to(torch.bfloat16)
    w[0, 3, :128] = 0
    bits = w.view(torch.int16).numpy().view(np.uint16)
    q4, s16 = oracle.quant_weight_int4(bits)
    assert q4.shape == (2, 8, 128) and s16.shape == (2, 8, 2)
    s = oracle.fp16_bits_to_f64(s16)
    assert s[0, 3, 0] == 1.0
    q = oracle.unpack_int4(q4).astype(np.int64)
    assert q.min() >= 0 and q.max() <= 15
    wf = oracle.bf16_bits_to_f64(bits)
    deq = oracle.dequant_weight_int4(q4, s16)
    srep = np.repeat(s, 128, axis=2)
    # non-clipped values round to the nearest multiple of the scale
    inner = (q > 0) & (q < 15)
    assert (np.abs(deq - wf)[inner] <= 0.5 * srep[inner] * (1 + 1e-6)).all()
    # the largest magnitude of each group maps to +-7 (or -8 never, since amax/7 scaling)
    amax_idx = np.abs(wf.reshape(2, 8, 2, 128)).argmax(axis=3)
    qq = q.reshape(2, 8, 2, 128)
    top = np.take_along_axis(qq, amax_idx[..., None], axis=3)[..., 0]
    nz = oracle.bf16_bits_to_f64(bits).reshape(2, 8, 2, 128).__abs__().max(axis=3) > 0
    assert set(np.unique(np.abs(top[nz] - 8))) <= {6, 7}
