"""GPU SwiGLU + 1x128 FP8 requantisation (moe_swiglu_quant) vs the oracle (the bar is that of
gpu_helpers.check_swiglu_quant: codes and scales equal to the float64 oracle's except within fp32 error of a
rounding boundary, every value within the E4M3 rounding bound, rows outside the segments untouched).
"""

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import oracle
from gpu_helpers import DEV, bf16_from_u16, check_swiglu_quant, require_gpu, u16

pytestmark = pytest.mark.gpu
SENT = 0xA5


def _run(gu_bits, layout, am, counts, seg, E):
    rows = gu_bits.shape[0]
    I = gu_bits.shape[1] // 2
    q = torch.full((rows, I), SENT, dtype=torch.uint8, device=DEV)
    sf = torch.full((rows, I // 128), -3.0, dtype=torch.float32, device=DEV)
    moe.moe_swiglu_quant(layout, bf16_from_u16(gu_bits), am, torch.from_numpy(counts.astype(np.int32)).to(DEV),
                         torch.from_numpy(seg.astype(np.int32)).to(DEV), E, q, sf)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy()


def _valid_rows(counts, seg, rows, layout, am):
    v = np.zeros(rows, bool)
    for e, c in enumerate(counts):
        st = e * am if layout == moe.LAYOUT_MASKED else int(seg[e])
        cap = am if layout == moe.LAYOUT_MASKED else rows - st
        v[st:st + max(0, min(int(c), cap))] = True
    return v


def _check(gu_bits, q, sf, valid):
    return check_swiglu_quant(gu_bits[valid], q, sf, valid, SENT, -3.0)


def _gu(rng, rows, I, scale=2.0):
    x = (rng.standard_normal((rows, 2 * I)) * scale).astype(np.float32)
    return oracle.f32_to_bf16_bits(x)


@pytest.mark.parametrize("I", [128, 384, 1536])
def test_swiglu_quant_contiguous_ragged(I):
    require_gpu()
    rng = np.random.default_rng(I)
    counts = np.array([0, 1, 17, 130, 0, 300, 5])
    E = len(counts)
    seg = np.zeros(E + 1, np.int64)
    for e in range(E):
        seg[e + 1] = seg[e] + -(-counts[e] // 128) * 128
    rows = int(seg[E]) + 128  # a tail past the last segment
    gu = _gu(rng, rows, I)
    q, sf = _run(gu, moe.LAYOUT_CONTIGUOUS, rows, counts, seg, E)
    _check(gu, q, sf, _valid_rows(counts, seg, rows, moe.LAYOUT_CONTIGUOUS, rows))


def test_swiglu_quant_masked_with_clipping_and_edge_values():
    require_gpu()
    rng = np.random.default_rng(9)
    E, max_m, I = 5, 24, 256
    counts = np.array([3, 0, 24, 40, 1])  # expert 3 is clipped to its 24 rows
    rows = E * max_m
    x = (rng.standard_normal((rows, 2 * I)) * 4).astype(np.float32)
    x[0, :I] = -100.0            # gate far negative: exp overflows, h = -0 * up
    x[1, :I] = 0.0               # gate zero: h = 0 (block amax 0 -> scale 1)
    x[2, I:] = 0.0               # up zero
    x[48, :] = 3e4               # large values: big scales
    x[49, :] = 1e-15             # tiny values: small scales
    gu = oracle.f32_to_bf16_bits(x)
    seg = np.arange(E + 1) * max_m
    q, sf = _run(gu, moe.LAYOUT_MASKED, max_m, counts, seg, E)
    valid = _valid_rows(counts, seg, rows, moe.LAYOUT_MASKED, max_m)
    _check(gu, q, sf, valid)
    assert (sf[1] == 1.0).all() and ((q[1] & 0x7F) == 0).all()  # +0 or -0 (the sign of up)


def test_swiglu_quant_qwen3_shape_and_determinism():
    require_gpu()
    import synth

    cfg = synth.config_by_name("qwen3_skewed")
    ids, _ = synth.route_inputs(cfg)
    r = oracle.route(ids.numpy(), cfg.E, "contiguous", align=cfg.align)
    rows, I = r["rows_cap"], cfg.K_down
    g = torch.Generator(device=DEV)
    g.manual_seed(synth.seed_for(cfg.index, 11))
    gu_t = (torch.randn(rows, 2 * I, generator=g, device=DEV) * 2).to(torch.bfloat16)
    counts = r["counts"]
    seg = r["seg_offsets"]
    q = torch.empty(rows, I, dtype=torch.uint8, device=DEV)
    sf = torch.empty(rows, I // 128, dtype=torch.float32, device=DEV)
    args = (moe.LAYOUT_CONTIGUOUS, gu_t, rows, torch.from_numpy(counts.astype(np.int32)).to(DEV),
            torch.from_numpy(seg.astype(np.int32)).to(DEV), cfg.E, q, sf)
    moe.moe_swiglu_quant(*args)
    torch.cuda.synchronize()
    q0, s0 = q.clone(), sf.clone()
    for _ in range(20):
        moe.moe_swiglu_quant(*args)
    torch.cuda.synchronize()
    assert torch.equal(q, q0) and torch.equal(sf, s0)
    # sampled rows: the first and last rows of every segment and a stride through the big ones
    pick = []
    for e in range(cfg.E):
        c, st = int(counts[e]), int(seg[e])
        if c:
            pick += list(range(st, st + min(c, 3))) + list(range(st + max(0, c - 3), st + c))
            pick += list(range(st, st + c, 257))
    pick = np.unique(np.array(pick))
    sel = torch.from_numpy(pick).to(DEV)
    gu_bits = u16(gu_t[sel])
    _check(gu_bits, q[sel].cpu().numpy(), sf[sel].cpu().numpy(), np.ones(len(pick), bool))
