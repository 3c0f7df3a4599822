"""Randomised shapes for every grouped-GEMM format against the oracle.

Each case draws the expert count, the segment sizes (empty, a few rows, about a
tile, several tiles), N, K, the layout (contiguous 128-row-aligned or masked
with a random capacity, so some experts are clipped), the weight order (row-
major or fragment-packed) and the tiling hint, so the dispatch lands on every
tile kind of every format over shapes the dedicated tests do not pin.  Codes
and scales come from the oracle's quantisers; the GPU result is held to the
path's bar against the oracle's exact sum (calc_diff below 1e-3 for FP8, FP8 x
MXFP4 and INT8, 1e-2 for the 4-bit weights, 1e-5 for BF16, plus the per-element
bound), and rows outside the segments must stay untouched.
"""

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import oracle
import weight_layout as wl
from gpu_helpers import DEV, bf16_from_u16, gemm_tolerance_check, require_gpu, u16

pytestmark = pytest.mark.gpu
SENT = 0x7BAD
FORMATS = ["fp8", "fp4", "int8", "int4", "bf16"]
BARS = {"fp8": 1e-3, "fp4": 1e-3, "int8": 1e-3, "int4": 1e-2, "bf16": 1e-5}


def _shape(rng):
    E = int(rng.integers(1, 11))
    kinds = rng.choice(4, size=E, p=[0.15, 0.3, 0.35, 0.2])
    lo_hi = [(0, 1), (1, 21), (60, 201), (250, 401)]
    counts = np.array([int(rng.integers(*lo_hi[k])) for k in kinds])
    N = int(rng.choice([128, 256, 384, 512]))
    K = 128 * int(rng.integers(1, 17))
    masked = bool(rng.integers(0, 2))
    max_m = int(rng.integers(8, 321)) if masked else 0
    packed = bool(rng.integers(0, 2))
    em = int(rng.choice([0, 1, 16, 48, 64, 128, 192, 256]))
    return E, counts, N, K, masked, max_m, packed, em


def _segments(counts, masked, max_m):
    E = len(counts)
    if masked:
        return np.arange(E + 1) * max_m, E * max_m, np.minimum(counts, max_m)
    starts = np.zeros(E + 1, np.int64)
    for e in range(E):
        starts[e + 1] = starts[e] + -(-counts[e] // 128) * 128
    return starts, max(int(starts[E]), 128), counts.copy()


def _bits(x):
    return oracle.f32_to_bf16_bits(np.asarray(x, np.float32))


def _run(fmt, seed):
    rng = np.random.default_rng(1000 + seed * 7 + FORMATS.index(fmt))
    E, counts, N, K, masked, max_m, packed, em = _shape(rng)
    print(f"[random gemm] {fmt} seed {seed}: E={E} counts={counts.tolist()} N={N} K={K} "
          f"{'masked max_m=' + str(max_m) if masked else 'contiguous'} packed={packed} expected_m={em}", flush=True)
    starts, rows, eff = _segments(counts, masked, max_m)
    layout = (moe.LAYOUT_MASKED if masked else moe.LAYOUT_CONTIGUOUS) | (moe.WEIGHTS_PACKED if packed else 0)
    am = max_m if masked else rows
    xb = _bits(rng.standard_normal((rows, K)))
    wb = _bits(rng.standard_normal((E, N, K)) * 0.02)
    D = torch.full((rows, N), SENT, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    cnt = torch.from_numpy(counts.astype(np.int32)).to(DEV)
    seg = torch.from_numpy(starts.astype(np.int32)).to(DEV)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    if fmt in ("fp8", "fp4"):
        a, sa = oracle.quant_act(xb)
        if fmt == "fp8":
            w, sw = oracle.quant_weight_fp8(wb)
            ref = oracle.grouped_gemm_fp8(a, sa, w, sw, eff, starts)
            wg = wl.pack_weight_fp8(w).reshape(w.shape) if packed else w
            moe.moe_grouped_gemm_fp8(layout, dev(a), dev(sa), dev(wg), dev(sw), D, cnt, seg, E, am, N, K, em)
        else:
            w4, s8 = oracle.quant_weight_fp4(wb)
            ref = oracle.grouped_gemm_fp8_fp4(a, sa, w4, s8, eff, starts)
            if packed:
                w4g, s8g = wl.pack_weight_fp4(w4, s8)
                w4g, s8g = w4g.reshape(w4.shape), s8g.reshape(s8.shape)
            else:
                w4g, s8g = w4, s8
            moe.moe_grouped_gemm_fp8_fp4(layout, dev(a), dev(sa), dev(w4g), dev(s8g), D, cnt, seg, E, am, N, K, em)
    elif fmt == "int8":
        a, sa = oracle.quant_int8(xb)
        w, sw = oracle.quant_int8(wb)
        ref = oracle.grouped_gemm_int8(a, sa, w, sw, eff, starts)
        wg = wl.pack_weight_fp8(w.view(np.uint8)).reshape(w.shape).view(np.int8) if packed else w
        moe.moe_grouped_gemm_int8(layout, dev(a), dev(sa), dev(wg), dev(sw.transpose(0, 2, 1)), D, cnt, seg, E, am,
                                  N, K, em)
    elif fmt == "int4":
        q4, s16 = oracle.quant_weight_int4(wb)
        ref = oracle.grouped_gemm_int4(xb, q4, s16, eff, starts)
        if packed:
            q4g, s16g = wl.pack_weight_int4(q4, s16)
            q4g, s16g = q4g.reshape(q4.shape), s16g.reshape(s16.shape)
        else:
            q4g, s16g = q4, s16
        S16 = torch.from_numpy(np.ascontiguousarray(s16g).view(np.int16)).view(torch.float16).to(DEV)
        moe.moe_grouped_gemm_int4(layout, bf16_from_u16(xb), dev(q4g), S16, D, cnt, seg, E, am, N, K, em)
    else:
        ref = oracle.grouped_gemm_bf16(xb, wb, eff, starts)
        wg = wl.pack_weight_bf16(wb).reshape(wb.shape) if packed else wb
        moe.moe_grouped_gemm_bf16(layout, bf16_from_u16(xb), bf16_from_u16(wg), D, cnt, seg, E, am, N, K, em)
    torch.cuda.synchronize()
    valid = np.isfinite(ref[:, 0])
    bits = u16(D)
    assert (bits[~valid] == SENT).all(), "rows outside the segments were written"
    if valid.any():
        gemm_tolerance_check(oracle.bf16_bits_to_f64(bits[valid]), ref[valid], BARS[fmt])


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("fmt", FORMATS)
def test_random_shapes_against_the_oracle(fmt, seed):
    require_gpu()
    _run(fmt, seed)
