"""GPU up-projection with SwiGLU and the 1x128 requantisation in its epilogue (moe_grouped_gemm_fp8_swiglu).

Its result is defined as the GEMM's bf16 output (gate columns 0 .. I-1, up columns I .. 2I-1) followed by
SwiGLU and the requantisation.  The oracle side: the float64 grouped GEMM, rounded to bf16, then the oracle's
SwiGLU and 1x128 quantisation.

  * Integer-valued operands with power-of-two scales make every partial sum exact in fp32, so the GPU's bf16
    gate/up values equal the oracle's; the codes and scales are then held to the SwiGLU bar
    (gpu_helpers.check_swiglu_quant), for every row-tile count of both tall tiles, both layouts and both weight
    orders, with rows outside the segments untouched.
  * Random FP8 operands: every output within the E4M3 rounding bound of the oracle's h, widened by what one
    bf16 rounding step of gate and up can move h (the GPU's fp32 accumulation may round to the neighbouring
    bf16); and bit-for-bit the result of the two-kernel chain moe_grouped_gemm_fp8 -> moe_swiglu_quant.
"""

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import oracle
import weight_layout as wl
from gpu_helpers import DEV, check_swiglu_quant, require_gpu

pytestmark = pytest.mark.gpu
SENT_Q, SENT_SF = 0xA5, -3.0


def _segments(counts, layout, max_m=0):
    E = len(counts)
    if layout == moe.LAYOUT_MASKED:
        starts = np.arange(E + 1) * max_m
        return starts, E * max_m, np.minimum(counts, max_m)
    starts = np.zeros(E + 1, np.int64)
    for e in range(E):
        starts[e + 1] = starts[e] + -(-counts[e] // 128) * 128
    return starts, max(int(starts[E]), 128), np.array(counts)


def _pow2(rng, shape, lo, hi):
    return np.exp2(rng.integers(lo, hi + 1, size=shape)).astype(np.float32)


def _int_codes(rng, shape, lo=-2, hi=2):
    """E4M3 codes of small integers (exact products and sums)."""
    code_of = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}
    v = rng.integers(lo, hi + 1, size=shape)
    mag = np.vectorize(lambda t: code_of[abs(int(t))])(v).astype(np.uint8)
    return np.where(v < 0, mag | 0x80, mag).astype(np.uint8)


def _run(c, packed, expected_m, chain=False):
    """The fused call (and, with chain, the two-kernel chain on the same inputs) -> numpy outputs."""
    E, I, K, rows = c["E"], c["I"], c["K"], c["rows"]
    A = torch.from_numpy(c["a"]).to(DEV)
    SFA = torch.from_numpy(c["sfa"]).to(DEV)
    wbytes = wl.pack_weight_fp8(c["w"]).reshape(c["w"].shape) if packed else c["w"]
    W = torch.from_numpy(np.ascontiguousarray(wbytes)).to(DEV)
    SFW = torch.from_numpy(c["sfw"]).to(DEV)
    counts = torch.from_numpy(c["counts"].astype(np.int32)).to(DEV)
    seg = torch.from_numpy(c["starts"].astype(np.int32)).to(DEV)
    am = c["max_m"] if c["layout"] == moe.LAYOUT_MASKED else rows
    layout = c["layout"] | (moe.WEIGHTS_PACKED if packed else 0)
    Q = torch.full((rows, I), SENT_Q, dtype=torch.uint8, device=DEV)
    SQ = torch.full((rows, I // 128), SENT_SF, dtype=torch.float32, device=DEV)
    print(f"[swiglu gemm] E={E} I={I} K={K} rows={rows} layout={c['layout']} packed={packed} em={expected_m}",
          flush=True)
    moe.moe_grouped_gemm_fp8_swiglu(layout, A, SFA, W, SFW, Q, SQ, counts, seg, E, am, I, K, expected_m)
    out = [Q, SQ]
    if chain:
        D = torch.empty(rows, 2 * I, dtype=torch.bfloat16, device=DEV)
        moe.moe_grouped_gemm_fp8(layout, A, SFA, W, SFW, D, counts, seg, E, am, 2 * I, K, expected_m)
        Qc = torch.full((rows, I), SENT_Q, dtype=torch.uint8, device=DEV)
        SQc = torch.full((rows, I // 128), SENT_SF, dtype=torch.float32, device=DEV)
        moe.moe_swiglu_quant(c["layout"], D, am, counts, seg, E, Qc, SQc)
        out += [Qc, SQc]
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _int_case(seed, counts, I, K, layout, max_m=0):
    rng = np.random.default_rng(seed)
    counts = np.array(counts)
    E = len(counts)
    starts, rows, eff = _segments(counts, layout, max_m)
    return dict(E=E, I=I, K=K, rows=rows, starts=starts, eff=eff, counts=counts, layout=layout, max_m=max_m,
                a=_int_codes(rng, (rows, K)), sfa=_pow2(rng, (rows, K // 128), -2, 1),
                w=_int_codes(rng, (E, 2 * I, K)), sfw=_pow2(rng, (E, 2 * I // 128, K // 128), -3, 0))


def _oracle_gate_up(c):
    ref = oracle.grouped_gemm_fp8(c["a"], c["sfa"], c["w"], c["sfw"], c["eff"], c["starts"])
    valid = np.isfinite(ref[:, 0])
    return ref, valid


# Integer operands put many h = silu(g) * u next to an E4M3 midpoint: for g above about 17, 1 + exp(-g) is 1 in
# fp32, so the GPU's h is exactly g * u (a short dyadic number, often a midpoint itself, rounded to even) while
# the float64 value lies a hair below it.  The SwiGLU bar's exceptions are then not rare; they are still
# required to be such near-midpoint cases.
_TIES = 2e-3

# rows per expert that give every row-tile count of the 256-row tile (2 .. 8 tiles of 32, the minimum 2 for
# one row) and of the 192-row tile (2 .. 6), plus experts of several tiles with ragged tails
_RAGGED = [0, 1, 33, 65, 97, 129, 161, 193, 225, 256, 0, 300, 450, 5]


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 128])  # 256-row and 192-row tall tiles
@pytest.mark.parametrize("I,K", [(128, 512), (384, 1024)])
def test_swiglu_gemm_integer_inputs_contiguous(I, K, expected_m, packed):
    require_gpu()
    c = _int_case(I + K + expected_m, _RAGGED, I, K, moe.LAYOUT_CONTIGUOUS)
    ref, valid = _oracle_gate_up(c)
    q, sq = _run(c, packed, expected_m)
    gu_bits = oracle.f64_to_bf16_bits(ref[valid])  # exact sums, rounded as the GEMM's bf16 output
    check_swiglu_quant(gu_bits, q, sq, valid, SENT_Q, SENT_SF, _TIES)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 100])
def test_swiglu_gemm_integer_inputs_masked_with_clipping(expected_m, packed):
    require_gpu()
    c = _int_case(7, [0, 5, 320, 999, 64], 256, 512, moe.LAYOUT_MASKED, max_m=320)
    ref, valid = _oracle_gate_up(c)
    q, sq = _run(c, packed, expected_m)
    check_swiglu_quant(oracle.f64_to_bf16_bits(ref[valid]), q, sq, valid, SENT_Q, SENT_SF, _TIES)


def test_swiglu_gemm_integer_inputs_degenerate_counts():
    """Every expert empty (nothing written), and counts past the segment (clipped to the rows there are)."""
    require_gpu()
    c = _int_case(8, [0, 0, 0], 128, 512, moe.LAYOUT_CONTIGUOUS)
    q, sq = _run(c, True, 0)
    assert (q == SENT_Q).all() and (sq == SENT_SF).all()
    c = _int_case(9, [40, 200], 128, 512, moe.LAYOUT_CONTIGUOUS)
    c["counts"] = np.array([40, 5000])  # the last segment holds 256 rows
    c["eff"] = np.array([40, 256])
    ref, valid = _oracle_gate_up(c)
    q, sq = _run(c, False, 0)
    check_swiglu_quant(oracle.f64_to_bf16_bits(ref[valid]), q, sq, valid, SENT_Q, SENT_SF, _TIES)


def _random_case(seed, counts, I, K, layout, max_m=0):
    rng = np.random.default_rng(seed)
    counts = np.array(counts)
    E = len(counts)
    starts, rows, eff = _segments(counts, layout, max_m)
    x = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((E, 2 * I, K)) * 0.05).astype(np.float32)).to(torch.bfloat16)
    u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    a, sfa = oracle.quant_act(u16(x))
    wq, sfw = oracle.quant_weight_fp8(u16(w))
    return dict(E=E, I=I, K=K, rows=rows, starts=starts, eff=eff, counts=counts, layout=layout, max_m=max_m,
                a=a, sfa=sfa, w=wq, sfw=sfw)


def _check_random(c, q, sq, valid, ref):
    """Every output within the E4M3 rounding bound of the oracle's h = silu(g) * u of the bf16-rounded exact
    gate/up values, widened by what the GPU's gate and up values may differ from those: its fp32 sum of the
    scaled products (error at most 2^-16 of the sum of their magnitudes here, generously) rounded to bf16 may
    land on the neighbouring bf16 (2^-7 relative).  Block scales within a factor 2 of the oracle's."""
    I = c["I"]
    assert (q[~valid] == SENT_Q).all() and (sq[~valid] == SENT_SF).all()
    gu = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(ref[valid]))
    mag = oracle.grouped_gemm_fp8(c["a"] & 0x7F, c["sfa"], c["w"] & 0x7F, c["sfw"], c["eff"], c["starts"])[valid]
    eps = 2.0 ** -16 * mag
    g, u = gu[:, :I], gu[:, I:]
    dg, du = 2.0 ** -7 * np.abs(g) + eps[:, :I], 2.0 ** -7 * np.abs(u) + eps[:, I:]
    h = oracle.swiglu(gu)
    qo, so = oracle.quant_act_values(h)
    sg = sq[valid]
    assert np.isin(sg / so, [0.5, 1.0, 2.0]).all()
    deq = oracle.dequant_act(q[valid], sg)
    s = np.repeat(sg.astype(np.float64), 128, axis=1)
    sil = oracle.silu(g)
    sig = 0.5 * (1.0 + np.tanh(0.5 * g))
    dsil = sig + 0.25 * (np.abs(g) + dg)  # |silu'| on [g - dg, g + dg]: sig + |x| sig (1 - sig), sig (1 - sig) <= 1/4
    move = dsil * dg * (np.abs(u) + du) + np.abs(sil) * du
    # (+ the fp32 evaluation of silu(g) * u: a few ulps)
    bound = (np.maximum(2.0 ** -4 * (np.abs(h) + move), 2.0 ** -10 * s) + move) * (1 + 1e-6) + 1e-6 * np.abs(h)
    err = np.abs(deq - h)
    i = np.unravel_index(np.argmax(err - bound), err.shape)
    assert (err <= bound).all(), (f"row {i[0]} col {i[1]}: g={g[i[0], i[1] % I]} u={u[i[0], i[1] % I]} h={h[i]} "
                                  f"deq={deq[i]} bound={bound[i]} scale={s[i]}")
    # the codes agree with the oracle's nearly everywhere (exceptions: a bf16 step or an E4M3 midpoint apart)
    assert np.mean(q[valid] == qo) > 0.99


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 128])
def test_swiglu_gemm_random_matches_oracle_and_the_two_kernel_chain(expected_m, packed):
    require_gpu()
    c = _random_case(11 + expected_m, _RAGGED, 256, 1024, moe.LAYOUT_CONTIGUOUS)
    ref, valid = _oracle_gate_up(c)
    q, sq, qc, sqc = _run(c, packed, expected_m, chain=True)
    assert np.array_equal(q, qc) and np.array_equal(sq, sqc)
    _check_random(c, q, sq, valid, ref)


def test_swiglu_gemm_masked_random_matches_the_two_kernel_chain_and_is_deterministic():
    require_gpu()
    c = _random_case(12, [3, 0, 500, 77], 384, 2048, moe.LAYOUT_MASKED, max_m=512)
    ref, valid = _oracle_gate_up(c)
    q, sq, qc, sqc = _run(c, True, 0, chain=True)
    assert np.array_equal(q, qc) and np.array_equal(sq, sqc)
    _check_random(c, q, sq, valid, ref)
    for _ in range(5):
        q2, sq2 = _run(c, True, 0)
        assert np.array_equal(q2, q) and np.array_equal(sq2, sq)
