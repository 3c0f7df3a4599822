"""GPU INT8 (1, 1, 128) quantisers and grouped GEMM vs the oracle.

Quantisation is bit-exact: the code is decided by the same correctly rounded
fp32 division on both sides.  The GEMM sums each 128-wide K block exactly in
int32 and promotes it with one fp32 product of the two scales and one fused
multiply-add, so against the oracle's exact sum y every element obeys

    |D - y| <= 2^-8 (|y| + err) + err,   err = (K/128 + 1) 2^-24 sum_kb |sa sw I_kb|

(I_kb the block's integer dot product; 2^-8 the unit roundoff of bf16's 8-bit
significand), checked
element by element next to the path's calc_diff / elementwise bar.  Where the
exact result is representable (small integer codes, power-of-two scales) the
GPU must match it bit for bit: one-hot activation rows (which pin how K, the
two 64-wide instructions per block and the per-channel scale columns line up)
and small integers.
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


def _bf16_bits(x):
    return oracle.f32_to_bf16_bits(np.asarray(x, np.float32))


def _quant_act_gpu(bits):
    rows, K = bits.shape
    q = torch.empty(rows, K, dtype=torch.int8, device=DEV)
    s = torch.empty(rows, K // 128, dtype=torch.float32, device=DEV)
    moe.moe_quant_act_int8(bf16_from_u16(bits), q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def _edge_rows(K):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((12, K)) * 3.0).astype(np.float32)
    x[0, :128] = 0.0                                   # all-zero block: s = 1, codes 0
    x[1, :] *= 1e30                                    # large magnitudes
    x[2, :] *= 1e-30                                   # tiny magnitudes
    x[3, :128] = np.float32(2.0 ** -133) * np.arange(128)  # bf16 subnormals: s itself is an fp32 subnormal
    x[4, :128] = -np.abs(x[4, :128])                   # one-signed block
    x[5, :128] = 0.0
    x[5, 7] = -1.0                                     # a single nonzero: it gets code -127
    # codes at exact halves: amax 127 gives s = 1, so x = j + 0.5 ties to even
    x[6, :128] = np.arange(128) - 63.5
    x[6, 0] = 127.0
    x[7, 128:256] = np.float32(1e-40)                  # one subnormal value repeated
    return x


def test_quant_act_int8_bit_exact():
    require_gpu()
    K = 640
    rng = np.random.default_rng(1)
    x = np.concatenate([_edge_rows(K), rng.standard_normal((301, K)).astype(np.float32)])
    bits = _bf16_bits(x)
    gq, gs = _quant_act_gpu(bits)
    oq, os_ = oracle.quant_int8(bits)
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(gq, oq)


def test_quant_act_int8_near_ties_bit_exact():
    """Many blocks with non-power-of-two scales: a few hundred codes whose quotient x / s lies within 2^-15 of a
    half-integer (where the kernel re-divides instead of multiplying by the rounded reciprocal) plus every other
    code, against the oracle's correctly rounded fp32 quotients; heavy-tailed values spread the scales."""
    require_gpu()
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((20000, 256)) * np.exp(rng.standard_normal((20000, 1)) * 4)).astype(np.float32)
    bits = _bf16_bits(x)
    gq, gs = _quant_act_gpu(bits)
    oq, os_ = oracle.quant_int8(bits)
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(gq, oq)
    xf = oracle.bf16_bits_to_f64(bits).astype(np.float32).reshape(20000, 2, 128)
    y = (xf / os_[..., None]).astype(np.float32)
    near = np.abs(y - (np.floor(y) + 0.5)) <= 2.0 ** -15
    assert near.sum() > 50, "the draw should exercise the re-division"


def test_quant_weight_int8_bit_exact_k_block_major_scales():
    require_gpu()
    rng = np.random.default_rng(2)
    E, N, K = 3, 256, 384
    w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    w[0, :12] = _edge_rows(K)
    bits = _bf16_bits(w)
    q = torch.empty(E, N, K, dtype=torch.int8, device=DEV)
    sw = torch.empty(E, K // 128, N, dtype=torch.float32, device=DEV)
    moe.moe_quant_weight_int8(bf16_from_u16(bits.reshape(E * N, K)).view(E, N, K), q, sw)
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_int8(bits)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), os_.transpose(0, 2, 1).view(np.uint32))


def _segments(counts, layout, max_m):
    E = len(counts)
    if layout == moe.LAYOUT_MASKED:
        return np.arange(E + 1) * max_m, E * max_m, np.minimum(counts, max_m)
    starts = np.zeros(E + 1, np.int64)
    for e in range(E):
        starts[e + 1] = starts[e] + -(-counts[e] // 128) * 128
    return starts, max(int(starts[E]), 128), np.array(counts)


def _case(seed, counts, N, K, layout, max_m=0, ints=False):
    rng = np.random.default_rng(seed)
    E = len(counts)
    starts, rows, eff = _segments(counts, layout, max_m)
    if ints:
        a = rng.integers(-4, 5, (rows, K)).astype(np.int8)
        sa = np.exp2(rng.integers(-2, 3, (rows, K // 128))).astype(np.float32)
        w = rng.integers(-4, 5, (E, N, K)).astype(np.int8)
        sw = np.exp2(rng.integers(-2, 3, (E, N, K // 128))).astype(np.float32)
    else:
        a, sa = oracle.quant_int8(_bf16_bits(rng.standard_normal((rows, K))))
        w, sw = oracle.quant_int8(_bf16_bits(rng.standard_normal((E, N, K)) * 0.02))
    return dict(E=E, N=N, K=K, rows=rows, starts=starts, eff=eff, counts=np.array(counts, np.int32), layout=layout,
                max_m=max_m, a=a, sa=sa, w=w, sw=sw)


def _run(c, expected_m=0, packed=False):
    """packed: the weight codes go in moe_pack_weight_fp8's order (the test helper's definition of it)."""
    D = torch.full((c["rows"], c["N"]), SENT, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    am = c["max_m"] if c["layout"] == moe.LAYOUT_MASKED else c["rows"]
    w = c["w"]
    if packed:
        w = wl.pack_weight_fp8(w.view(np.uint8)).reshape(w.shape).view(np.int8)
    layout = c["layout"] | (moe.WEIGHTS_PACKED if packed else 0)
    moe.moe_grouped_gemm_int8(layout, torch.from_numpy(c["a"]).to(DEV), torch.from_numpy(c["sa"]).to(DEV),
                              torch.from_numpy(np.ascontiguousarray(w)).to(DEV),
                              torch.from_numpy(np.ascontiguousarray(c["sw"].transpose(0, 2, 1))).to(DEV), D,
                              torch.from_numpy(c["counts"]).to(DEV),
                              torch.from_numpy(c["starts"].astype(np.int32)).to(DEV), c["E"], am, c["N"], c["K"],
                              expected_m)
    torch.cuda.synchronize()
    return D


def _ref(c):
    return oracle.grouped_gemm_int8(c["a"], c["sa"], c["w"], c["sw"], c["eff"], c["starts"])


def _abs_block_sum(c, valid_rows):
    """sum_kb |sa sw I_kb| for every valid row (float64)."""
    K, N = c["K"], c["N"]
    out = np.zeros((len(valid_rows), N))
    e_of = np.zeros(c["rows"], np.int64)
    for e in range(c["E"]):
        e_of[c["starts"][e]:c["starts"][e] + c["eff"][e]] = e
    for kb in range(K // 128):
        ab = c["a"][valid_rows, 128 * kb:128 * kb + 128].astype(np.int64)
        sa = c["sa"][valid_rows, kb].astype(np.float64)
        for e in np.unique(e_of[valid_rows]):
            m = e_of[valid_rows] == e
            wb = c["w"][e, :, 128 * kb:128 * kb + 128].astype(np.int64)
            blk = ab[m] @ wb.T
            out[m] += np.abs(blk * sa[m, None] * c["sw"][e, :, kb].astype(np.float64)[None, :])
    return out


def _check(c, D, exact=False):
    ref = _ref(c)
    valid = np.isfinite(ref[:, 0])
    bits = u16(D)
    assert (bits[~valid] == SENT).all(), "rows outside the segments were written"
    got = oracle.bf16_bits_to_f64(bits[valid])
    if exact:
        want = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits_normal(ref[valid]))
        assert np.array_equal(got, want)
        return
    y = ref[valid]
    err = (c["K"] // 128 + 1) * 2.0 ** -24 * _abs_block_sum(c, np.nonzero(valid)[0])
    excess = np.abs(got - y) - (2.0 ** -8 * (np.abs(y) + err) + err)
    assert excess.max() <= 0.0, f"fp32 accumulation bound exceeded by {excess.max():.3e}"
    gemm_tolerance_check(got, y, 1e-3)


@pytest.mark.parametrize("packed,expected_m", [(False, 16), (False, 64), (True, 16), (True, 64)])
def test_int8_one_hot_rows_pin_the_operand_layout(packed, expected_m):
    """Row r holds one nonzero code at k_r: D[r, n] = a * sa * w[n, k_r] * sw[n, k_r / 128], exact with power-of-two
    scales (distinct per column and K block, so a scale read from the wrong column or block changes the value)."""
    require_gpu()
    rng = np.random.default_rng(2)
    c = _case(2, [40], N=256, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    c["w"][:] = rng.integers(-127, 128, c["w"].shape).astype(np.int8)
    c["sw"][:] = np.exp2(rng.integers(-6, 7, c["sw"].shape)).astype(np.float32)
    ks = [0, 1, 15, 16, 31, 47, 63, 64, 65, 79, 95, 127, 128, 129, 200, 255, 300, 383, 384, 447, 510, 511]
    ks += list(range(17, 35))
    c["a"][:] = 0
    c["sa"][:] = np.exp2(rng.integers(-3, 4, c["sa"].shape)).astype(np.float32)
    codes = rng.choice([-127, -5, -1, 1, 3, 100, 127], size=40)
    for r, k in enumerate(ks[:40]):
        c["a"][r, k] = codes[r]
    bits = u16(_run(c, expected_m, packed))[:40]
    for r, k in enumerate(ks[:40]):
        y = float(codes[r]) * c["sa"][r, k // 128] * c["w"][0, :, k].astype(np.float64) * c["sw"][0, :, k // 128]
        want = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits_normal(y))
        assert np.array_equal(oracle.bf16_bits_to_f64(bits[r]), want), f"row {r}, k {k}"


@pytest.mark.parametrize("packed,expected_m", [(False, 0), (False, 16), (True, 16), (True, 64)])
def test_int8_small_integers_exact_and_deterministic(packed, expected_m):
    require_gpu()
    c = _case(5, [7, 64, 90, 129, 300], N=512, K=1024, layout=moe.LAYOUT_CONTIGUOUS, ints=True)
    D = _run(c, expected_m, packed)
    _check(c, D, exact=True)
    for _ in range(10):
        assert torch.equal(_run(c, expected_m, packed), D)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 16, 64])
def test_int8_contiguous_ragged(expected_m, packed):
    """Segments of 0, 1, 17, 80, 130 and 300 rows (every computed height of both tiles: 16-row units; 64, 96,
    128, 160 and 192 of the 192-row units), N = 384 (the second 256-column tile has idle waves), K/128 = 13 (ring
    wrap-arounds plus a tail)."""
    require_gpu()
    c = _case(3, [0, 1, 17, 80, 130, 300], N=384, K=1664, layout=moe.LAYOUT_CONTIGUOUS)
    _check(c, _run(c, expected_m, packed))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 16])
def test_int8_masked_clipped(expected_m, packed):
    """Masked segments; counts above max_m are clipped to it (rows past the capacity never written)."""
    require_gpu()
    c = _case(4, [5, 0, 64, 90, 1, 33], N=256, K=768, layout=moe.LAYOUT_MASKED, max_m=64)
    _check(c, _run(c, expected_m, packed))


@pytest.mark.parametrize("expected_m", [16, 64])
def test_int8_degenerate_shapes(expected_m):
    """K = 128 (one block, fewer than the ring depth), N = 128 (waves 2 and 3 idle), a single row, and a call
    whose experts are all empty (nothing written)."""
    require_gpu()
    c = _case(6, [1, 0, 3], N=128, K=128, layout=moe.LAYOUT_CONTIGUOUS)
    _check(c, _run(c, expected_m))
    c = _case(7, [0, 0, 0, 0], N=256, K=256, layout=moe.LAYOUT_CONTIGUOUS)
    assert (u16(_run(c, expected_m)) == SENT).all()
    c = _case(8, [1], N=256, K=7168, layout=moe.LAYOUT_MASKED, max_m=1)
    _check(c, _run(c, expected_m))


def test_int8_chain_quantise_then_gemm():
    """bf16 activations and weights quantised on the GPU, then multiplied: equal codes and scales to the oracle's,
    and the GEMM within the bound above of the oracle's chain; the chain's error against the unquantised bf16
    product is reported by the path's bar (calc_diff of INT8 (1, 1, 128) on both operands)."""
    require_gpu()
    rng = np.random.default_rng(9)
    E, N, K, counts = 4, 512, 2048, [33, 0, 150, 71]
    starts, rows, eff = _segments(counts, moe.LAYOUT_CONTIGUOUS, 0)
    xb = _bf16_bits(rng.standard_normal((rows, K)))
    wb = _bf16_bits(rng.standard_normal((E, N, K)) * 0.02)
    qa, sa = _quant_act_gpu(xb)
    qw = torch.empty(E, N, K, dtype=torch.int8, device=DEV)
    swt = torch.empty(E, K // 128, N, dtype=torch.float32, device=DEV)
    moe.moe_quant_weight_int8(bf16_from_u16(wb.reshape(E * N, K)).view(E, N, K), qw, swt)
    torch.cuda.synchronize()
    oa, osa = oracle.quant_int8(xb)
    ow, osw = oracle.quant_int8(wb)
    assert np.array_equal(qa, oa) and np.array_equal(sa, osa)
    assert np.array_equal(qw.cpu().numpy(), ow) and np.array_equal(swt.cpu().numpy(), osw.transpose(0, 2, 1))
    c = dict(E=E, N=N, K=K, rows=rows, starts=starts, eff=eff, counts=np.array(counts, np.int32),
             layout=moe.LAYOUT_CONTIGUOUS, max_m=0, a=oa, sa=osa, w=ow, sw=osw)
    D = _run(c, 64)
    _check(c, D)
    # against the unquantised product: INT8 on both sides stays well inside the path's bar
    ok = np.isfinite(_ref(c)[:, 0])
    xf = oracle.bf16_bits_to_f64(xb)
    wf = oracle.bf16_bits_to_f64(wb)
    full = np.full((rows, N), np.nan)
    for e in range(E):
        p0, n = int(starts[e]), int(eff[e])
        full[p0:p0 + n] = xf[p0:p0 + n] @ wf[e].T
    got = oracle.bf16_bits_to_f64(u16(D)[ok])
    assert oracle.calc_diff(got, full[ok]) < 1e-3
