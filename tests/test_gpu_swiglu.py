"""GPU SwiGLU + 1x128 FP8 requantisation (moe_swiglu_quant) vs the oracle.

The kernel evaluates h = silu(gate) * up in fp32 (expf, one IEEE division, one
multiply: a few fp32 ulps from the exact value) and the oracle in float64, so
a code or a scale can differ only where the float64 value lies within that
error of a rounding boundary of the E4M3 grid or of the power-of-two scale
rule.  The test therefore requires:
  * every scale a power of two, and equal to the oracle's unless the block's
    float64 amax is within 1e-6 (relative) of a boundary 448 * 2^k, or below
    the fp32 normal range (h underflows to 0 in fp32: zero codes either way);
  * every code equal to the oracle's unless the block's scale differs or the
    float64 scaled value is within 1e-6 (relative) of an E4M3 rounding
    midpoint -- and such exceptions to be rare;
  * every dequantised value within the E4M3 rounding bound of the float64 h;
  * rows outside the segments untouched.
"""

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import oracle
from gpu_helpers import DEV, bf16_from_u16, require_gpu, u16

pytestmark = pytest.mark.gpu
SENT = 0xA5


def _midpoints():
    """Sorted float64 midpoints between consecutive non-negative E4M3 values (0 .. 448)."""
    tab = oracle.e4m3_decode_table()[:127]
    return (tab[:-1] + tab[1:]) / 2.0


MID = _midpoints()


def _near_midpoint(v, rel=1e-6):
    a = np.abs(v)
    i = np.clip(np.searchsorted(MID, a), 1, len(MID) - 1)
    d = np.minimum(np.abs(a - MID[i - 1]), np.abs(a - MID[i]))
    return d <= rel * np.maximum(a, 2.0 ** -9)


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
    I = gu_bits.shape[1] // 2
    assert (q[~valid] == SENT).all() and (sf[~valid] == -3.0).all(), "rows outside the segments were written"
    gu = oracle.bf16_bits_to_f64(gu_bits[valid])
    h = oracle.swiglu(gu)
    qo, so = oracle.quant_act_values(h)
    qg, sg = q[valid], sf[valid]
    bits = sg.view(np.uint32)
    assert ((bits & 0x807FFFFF) == 0).all() and (bits != 0).all(), "scales must be powers of two"
    nb = I // 128
    amax = np.abs(h.reshape(-1, nb, 128)).max(axis=2)
    ratio = amax / 448.0
    near_scale = (ratio > 0) & (np.abs(ratio / np.exp2(np.round(np.log2(np.maximum(ratio, 1e-300)))) - 1.0) <= 1e-6)
    # a block whose float64 amax lies below the fp32 normal range underflows to 0 in fp32 (scale 1, zero codes)
    # while float64 keeps a tiny value (scale 2^-126, zero codes): the same zeros, encoded with another scale
    tiny = amax < 2.0 ** -120
    scale_ok = (sg == so) | near_scale | tiny
    assert scale_ok.all(), f"{int((~scale_ok).sum())} block scales differ away from a boundary"
    same_scale = np.repeat(sg == so, 128, axis=1)
    scaled = h / np.repeat(so.astype(np.float64), 128, axis=1)
    code_ok = (qg == qo) | ~same_scale | _near_midpoint(scaled)
    assert code_ok.all(), f"{int((~code_ok).sum())} codes differ away from a rounding midpoint"
    exceptions = int(((qg != qo) & same_scale).sum())
    assert exceptions <= max(2, qg.size // 10000), f"{exceptions} of {qg.size} codes differ"
    deq = oracle.dequant_act(qg, sg)
    s = np.repeat(sg.astype(np.float64), 128, axis=1)
    assert (np.abs(deq - h) <= np.maximum(2.0 ** -4 * np.abs(h), 2.0 ** -10 * s) * (1 + 1e-5) + 1e-30).all()
    return exceptions


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
