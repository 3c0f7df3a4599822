"""GPU grouped GEMMs (FP8 block-scaled, INT4 weight-only) vs the oracle."""

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import oracle
import weight_layout as wl
from gpu_helpers import DEV, bf16_from_u16, gemm_tolerance_check, require_gpu, u16

pytestmark = pytest.mark.gpu
SENT_BITS = 0x7BAD  # a bf16 pattern no GEMM result takes in these tests


def _layout_rows(counts, layout, align=128, max_m=0):
    E = len(counts)
    if layout == moe.LAYOUT_MASKED:
        starts = np.arange(E + 1) * max_m
        return starts, E * max_m, np.minimum(counts, max_m)
    starts = np.zeros(E + 1, np.int64)
    for e in range(E):
        starts[e + 1] = starts[e] + -(-counts[e] // align) * align
    return starts, int(starts[E]) if starts[E] > 0 else align, np.array(counts)


def _fp8_case(seed, counts, N, K, layout, max_m=0, act_scale=1.0):
    rng = np.random.default_rng(seed)
    E = len(counts)
    starts, rows, eff = _layout_rows(np.array(counts), layout, max_m=max_m)
    x = torch.from_numpy((rng.standard_normal((rows, K)) * act_scale).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    a_codes, sfa = oracle.quant_act(u16(x))
    w_codes, sfw = oracle.quant_weight_fp8(u16(w))
    return dict(E=E, N=N, K=K, rows=rows, starts=starts, eff=eff, counts=np.array(counts, np.int32), layout=layout,
                max_m=max_m, a=a_codes, sfa=sfa, w=w_codes, sfw=sfw)


def _run_fp8(c, expected_m=0, D=None, packed=False, sfa_shift=0):
    """packed: the weights go in the oracle's fragment-packed order, with MOE_WEIGHTS_PACKED.
    sfa_shift: place SFA that many floats into a larger buffer (a pointer that is only 4-byte aligned)."""
    A = torch.from_numpy(c["a"]).to(DEV)
    SFA = torch.from_numpy(c["sfa"]).to(DEV)
    if sfa_shift:
        buf = torch.zeros(SFA.numel() + sfa_shift, dtype=torch.float32, device=DEV)
        buf[sfa_shift:] = SFA.reshape(-1)
        SFA = buf[sfa_shift:].view(SFA.shape)
    wbytes = wl.pack_weight_fp8(c["w"]).reshape(c["w"].shape) if packed else c["w"]
    W = torch.from_numpy(np.ascontiguousarray(wbytes)).to(DEV)
    SFW = torch.from_numpy(c["sfw"]).to(DEV)
    if D is None:
        D = torch.full((c["rows"], c["N"]), SENT_BITS, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    counts = torch.from_numpy(c["counts"]).to(DEV)
    seg = torch.from_numpy(c["starts"].astype(np.int32)).to(DEV)
    am = c["max_m"] if c["layout"] == moe.LAYOUT_MASKED else c["rows"]
    layout = c["layout"] | (moe.WEIGHTS_PACKED if packed else 0)
    moe.moe_grouped_gemm_fp8(layout, A, SFA, W, SFW, D, counts, seg, c["E"], am, c["N"], c["K"], expected_m)
    torch.cuda.synchronize()
    return D


def _check_fp8(c, D):
    ref = oracle.grouped_gemm_fp8(c["a"], c["sfa"], c["w"], c["sfw"], c["eff"], c["starts"])
    valid = np.isfinite(ref[:, 0])
    got = D.float().cpu().numpy().astype(np.float64)
    gemm_tolerance_check(got[valid], ref[valid], 1e-3)
    # rows outside the segments are never written
    bits = u16(D)
    assert (bits[~valid] == SENT_BITS).all()


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 16, 64, 256])
def test_fp8_contiguous_ragged(expected_m, packed):
    require_gpu()
    # K = 1536: 12 K blocks, three row-scale groups of the tall tile
    c = _fp8_case(1, [0, 1, 17, 130, 300], N=384, K=1536, layout=moe.LAYOUT_CONTIGUOUS)
    _check_fp8(c, _run_fp8(c, expected_m, packed=packed))


@pytest.mark.parametrize("packed", [False, True])
def test_fp8_tall_sized_calls_the_tall_tile_cannot_take(packed):
    """K/128 not a multiple of 4, or SFA only 4-byte aligned: prefill-sized calls run on the 64-row tile."""
    require_gpu()
    c = _fp8_case(14, [0, 1, 17, 130, 300], N=384, K=640, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (0, 128, 256):
        _check_fp8(c, _run_fp8(c, em, packed=packed))
    c = _fp8_case(15, [70, 260, 0, 5], N=256, K=1024, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (0, 128):
        _check_fp8(c, _run_fp8(c, em, packed=packed, sfa_shift=1))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 16, 64])
def test_fp8_masked_with_overfull_expert(expected_m, packed):
    require_gpu()
    c = _fp8_case(2, [0, 20, 3, 17, 1, 25], N=256, K=384, layout=moe.LAYOUT_MASKED, max_m=20)
    _check_fp8(c, _run_fp8(c, expected_m, packed=packed))


@pytest.mark.parametrize("packed", [False, True])
def test_fp8_masked_tall_segments(packed):
    """Masked layout with segments taller than one tall tile (192 or 256 rows: several M chunks, ragged tails)."""
    require_gpu()
    c = _fp8_case(12, [150, 0, 300, 65], N=384, K=1024, layout=moe.LAYOUT_MASKED, max_m=300)
    for em in (0, 200, 256):
        _check_fp8(c, _run_fp8(c, em, packed=packed))


@pytest.mark.parametrize("packed", [False, True])
def test_fp8_tall_schedule_every_chunk_class(packed):
    """The unit table orders full chunks first, then partial chunks by size: 100 experts (several per lane of
    the table build), rows that are exact multiples of both tall heights, and partial chunks of every 32-row
    size class, on both tall tiles."""
    require_gpu()
    rng = np.random.default_rng(21)
    counts = [0, 192, 256, 384, 512, 768, 1000, 7, 33] + [32 * c - int(rng.integers(0, 32)) for c in range(1, 9)]
    counts += rng.integers(0, 600, size=100 - len(counts)).tolist()
    c = _fp8_case(21, counts, N=512, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (128, 256):
        _check_fp8(c, _run_fp8(c, em, packed=packed))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("K", [1536, 2560])
def test_fp8_tall_every_row_tile_count_long_k(K, packed):
    """Every row-tile count of both tall heights (units of 1..256 rows, so every loop body) with a K loop that
    has main iterations before its last one (K/128 = 12 or 20)."""
    require_gpu()
    counts = [32 * r - 5 for r in range(1, 9)] + [32 * r for r in range(1, 9)] + [0, 3, 256 + 100, 192 + 40]
    c = _fp8_case(51 + K, counts, N=256, K=K, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (128, 256):
        _check_fp8(c, _run_fp8(c, em, packed=packed))


@pytest.mark.parametrize("packed", [False, True])
def test_fp8_degenerate_expert_counts(packed):
    """No rows at all (an empty unit table), 1024 experts with 0..3 rows (16 experts per lane of the table
    build, every 4-bit size-class slot used; N = 128, so half of each tall tile's waves store nothing), and a
    single expert with several chunks, on every tile height."""
    require_gpu()
    for layout, mm in ((moe.LAYOUT_CONTIGUOUS, 0), (moe.LAYOUT_MASKED, 16)):
        c = _fp8_case(31, [0] * 8, N=256, K=512, layout=layout, max_m=mm)
        for em in (16, 64, 128, 256):
            _check_fp8(c, _run_fp8(c, em, packed=packed))
    counts = np.random.default_rng(33).integers(0, 4, size=1024).tolist()
    c = _fp8_case(33, counts, N=128, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (16, 128, 256):
        _check_fp8(c, _run_fp8(c, em, packed=packed))
    c = _fp8_case(34, [700], N=384, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (64, 128, 256):
        _check_fp8(c, _run_fp8(c, em, packed=packed))


@pytest.mark.parametrize("packed", [False, True])
def test_fp8_many_experts_long_k(packed):
    require_gpu()
    rng = np.random.default_rng(3)
    counts = rng.integers(0, 40, size=33).tolist()
    c = _fp8_case(3, counts, N=512, K=2560, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (24, 128):
        _check_fp8(c, _run_fp8(c, em, packed=packed))


def test_pack_weight_fp8_bit_exact():
    """The library's packed weight order equals the oracle's, byte for byte (two experts, ragged K blocks)."""
    require_gpu()
    rng = np.random.default_rng(13)
    q = rng.integers(0, 256, size=(2, 384, 640), dtype=np.uint8)
    out = torch.full(q.shape, 0x5A, dtype=torch.uint8, device=DEV)
    moe.moe_pack_weight_fp8(torch.from_numpy(q).to(DEV), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().reshape(2, -1), wl.pack_weight_fp8(q))


def _int_codes(rng, shape, lo=-4, hi=4):
    code_of = np.array([0x00, 0x38, 0x40, 0x44, 0x48], np.uint8)  # E4M3 codes of 0 .. 4
    v = rng.integers(lo, hi + 1, size=shape)
    codes = code_of[np.abs(v)] | np.where(v < 0, 0x80, 0).astype(np.uint8)
    return v, codes


def test_fp8_small_integers_bit_exact():
    """Integer-valued codes with unit scales: every partial sum is exact, so is the bf16 result."""
    require_gpu()
    rng = np.random.default_rng(4)
    E, N, K = 3, 256, 512
    counts = np.array([5, 0, 40], np.int32)
    starts = np.array([0, 128, 128, 256])
    av, a = _int_codes(rng, (256, K), -2, 2)
    wv, w = _int_codes(rng, (E, N, K), -2, 2)
    c = dict(E=E, N=N, K=K, rows=256, starts=starts, eff=counts, counts=counts, layout=moe.LAYOUT_CONTIGUOUS,
             max_m=0, a=a, sfa=np.ones((256, K // 128), np.float32), w=w, sfw=np.ones((E, N // 128, K // 128),
                                                                                          np.float32))
    # em 16 and 64: short tiles; 128: 192-row tall tiles; 0 (contiguous default) and 256: 256-row tall tiles
    for em, packed in ((0, False), (16, False), (64, False), (128, False), (0, True), (16, True), (128, True)):
        D = _run_fp8(c, em, packed=packed)
        for e in range(E):
            s, n = int(starts[e]), int(counts[e])
            exact = av[s:s + n] @ wv[e].T
            assert np.array_equal(u16(D)[s:s + n], oracle.f64_to_bf16_bits(exact.astype(np.float64)))


@pytest.mark.parametrize("packed", [False, True])
def test_fp8_tall_units_in_sequence_bit_exact(packed):
    """Several tall units per workgroup (each unit issues the next one's first K blocks before it ends), of
    every row-tile count in a row and with idle waves (N = 896: the last column tile has 128), on small-integer
    codes with power-of-two scales (every sum exact): each output must equal the integer product rounded to
    bf16."""
    require_gpu()
    rng = np.random.default_rng(8)
    E, N, K = 128, 896, 512
    counts = rng.integers(1, 520, size=E).astype(np.int32)
    starts, rows, _ = _layout_rows(counts, moe.LAYOUT_CONTIGUOUS)
    av, a = _int_codes(rng, (rows, K), -2, 2)
    wv, w = _int_codes(rng, (E, N, K), -2, 2)
    sa = np.exp2(rng.integers(-2, 2, size=(rows, K // 128))).astype(np.float32)
    sw = np.exp2(rng.integers(-2, 1, size=(E, N // 128, K // 128))).astype(np.float32)
    c = dict(E=E, N=N, K=K, rows=rows, starts=starts, eff=counts, counts=counts, layout=moe.LAYOUT_CONTIGUOUS,
             max_m=0, a=a, sfa=sa, w=w, sfw=sw)
    ref = np.zeros((rows, N), np.uint16)
    for e in range(E):
        s0, n = int(starts[e]), int(counts[e])
        av_e = (av[s0:s0 + n].reshape(n, K // 128, 128) * sa[s0:s0 + n, :, None]).reshape(n, K)
        wv_e = (wv[e].reshape(N, K // 128, 128) * np.repeat(sw[e], 128, axis=0)[:, :, None]).reshape(N, K)
        ref[s0:s0 + n] = oracle.f64_to_bf16_bits_normal(av_e.astype(np.float64) @ wv_e.astype(np.float64).T)
    for em in (128, 256):  # 192- and 256-row units: about 2 per workgroup
        D = u16(_run_fp8(c, em, packed=packed))
        for e in range(E):
            s0, n = int(starts[e]), int(counts[e])
            assert np.array_equal(D[s0:s0 + n], ref[s0:s0 + n]), (em, e)


def test_fp8_scale_invariance_bit_exact():
    require_gpu()
    c = _fp8_case(5, [9, 33], N=256, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    D0 = _run_fp8(c)
    c2 = dict(c)
    c2["sfa"] = c["sfa"] * np.float32(8.0)
    c2["sfw"] = c["sfw"] * np.float32(0.125)
    D1 = _run_fp8(c2)
    assert torch.equal(D0, D1)
    c3 = dict(c)
    c3["sfa"] = c["sfa"] * np.float32(4.0)
    D2 = _run_fp8(c3)
    valid = np.isfinite(oracle.grouped_gemm_fp8(c["a"], c["sfa"], c["w"], c["sfw"], c["eff"], c["starts"])[:, 0])
    assert torch.equal((D0.float() * 4)[torch.from_numpy(valid).to(DEV)], D2.float()[torch.from_numpy(valid).to(DEV)])


@pytest.mark.parametrize("packed", [False, True])
def test_fp8_determinism_20_runs(packed):
    require_gpu()
    c = _fp8_case(6, [50, 0, 200, 7], N=256, K=1024, layout=moe.LAYOUT_CONTIGUOUS)
    ref = _run_fp8(c, packed=packed)
    for _ in range(20):
        assert torch.equal(_run_fp8(c, packed=packed), ref)
    # the packed order changes the loads only, never the arithmetic
    assert torch.equal(_run_fp8(c, packed=not packed), ref)


# --------------------------------------------------------------------- INT4 --
def _int4_case(seed, counts, N, K, layout, max_m=0):
    rng = np.random.default_rng(seed)
    E = len(counts)
    starts, rows, eff = _layout_rows(np.array(counts), layout, max_m=max_m)
    x = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    q4, s16 = oracle.quant_weight_int4(u16(w))
    return dict(E=E, N=N, K=K, rows=rows, starts=starts, eff=eff, counts=np.array(counts, np.int32), layout=layout,
                max_m=max_m, a=u16(x), q4=q4, s16=s16)


def _run_int4(c, expected_m=0, packed=False):
    """packed: the weights go in the oracle's fragment-packed order, with MOE_WEIGHTS_PACKED."""
    A = bf16_from_u16(c["a"])
    wbytes, sbits = c["q4"], c["s16"]
    if packed:
        wbytes, sbits = wl.pack_weight_int4(c["q4"], c["s16"])
        wbytes, sbits = wbytes.reshape(c["q4"].shape), sbits.reshape(c["s16"].shape)
    W4 = torch.from_numpy(wbytes).to(DEV)
    S16 = torch.from_numpy(sbits.view(np.int16)).view(torch.float16).to(DEV)
    D = torch.full((c["rows"], c["N"]), SENT_BITS, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    counts = torch.from_numpy(c["counts"]).to(DEV)
    seg = torch.from_numpy(c["starts"].astype(np.int32)).to(DEV)
    am = c["max_m"] if c["layout"] == moe.LAYOUT_MASKED else c["rows"]
    layout = c["layout"] | (moe.WEIGHTS_PACKED if packed else 0)
    moe.moe_grouped_gemm_int4(layout, A, W4, S16, D, counts, seg, c["E"], am, c["N"], c["K"], expected_m)
    torch.cuda.synchronize()
    return D


def _check_int4(c, D):
    ref = oracle.grouped_gemm_int4(c["a"], c["q4"], c["s16"], c["eff"], c["starts"])
    valid = np.isfinite(ref[:, 0])
    got = D.float().cpu().numpy().astype(np.float64)
    gemm_tolerance_check(got[valid], ref[valid], 1e-2)
    assert (u16(D)[~valid] == SENT_BITS).all()


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 16])
def test_int4_masked(expected_m, packed):
    require_gpu()
    c = _int4_case(7, [0, 1, 16, 5, 9, 30], N=384, K=640, layout=moe.LAYOUT_MASKED, max_m=16)
    _check_int4(c, _run_int4(c, expected_m, packed=packed))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 16])
def test_int4_contiguous_ragged(expected_m, packed):
    require_gpu()
    c = _int4_case(8, [3, 0, 70, 129], N=256, K=1024, layout=moe.LAYOUT_CONTIGUOUS)
    _check_int4(c, _run_int4(c, expected_m, packed=packed))


@pytest.mark.parametrize("packed", [False, True])
def test_int4_long_k_restages_scales(packed):
    """130 K groups: the 64-row tile holds 128 groups of scales in LDS and restages once; 16-row tiles hold all."""
    require_gpu()
    c = _int4_case(12, [40, 0, 70], N=256, K=130 * 128, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (16, 64):
        _check_int4(c, _run_int4(c, em, packed=packed))


@pytest.mark.parametrize("packed", [False, True])
def test_int4_degenerate_expert_counts(packed):
    """No rows at all, 1024 experts with 0..2 rows, one expert with several M chunks."""
    require_gpu()
    c = _int4_case(41, [0] * 8, N=256, K=512, layout=moe.LAYOUT_MASKED, max_m=16)
    for em in (0, 16):
        _check_int4(c, _run_int4(c, em, packed=packed))
    counts = np.random.default_rng(42).integers(0, 3, size=1024).tolist()
    c = _int4_case(42, counts, N=128, K=256, layout=moe.LAYOUT_MASKED, max_m=2)
    _check_int4(c, _run_int4(c, 0, packed=packed))
    c = _int4_case(43, [300], N=256, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (0, 16):
        _check_int4(c, _run_int4(c, em, packed=packed))


def test_int4_packed_many_rows_and_partial_tiles():
    """Packed weights with up to 150 rows per expert (ten 16-row units) and N = 384 (a half-idle last tile)."""
    require_gpu()
    c = _int4_case(13, [150, 1, 0, 33, 17], N=384, K=384, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (0, 4, 128):
        _check_int4(c, _run_int4(c, em, packed=True))


def test_pack_weight_int4_bit_exact():
    """The library's packed 4-bit weights and scales equal the oracle's, bit for bit (two experts, three groups)."""
    require_gpu()
    rng = np.random.default_rng(14)
    q4 = rng.integers(0, 256, size=(2, 384, 192), dtype=np.uint8)
    s16 = rng.integers(0, 1 << 15, size=(2, 384, 3), dtype=np.uint16)
    qo = torch.full(q4.shape, 0x5A, dtype=torch.uint8, device=DEV)
    so = torch.full(s16.shape, 7, dtype=torch.int16, device=DEV).view(torch.float16)
    moe.moe_pack_weight_int4(torch.from_numpy(q4).to(DEV), torch.from_numpy(s16.view(np.int16)).to(DEV).view(torch.float16),
                             qo, so)
    torch.cuda.synchronize()
    wq, ws = wl.pack_weight_int4(q4, s16)
    assert np.array_equal(qo.cpu().numpy().reshape(2, -1), wq)
    assert np.array_equal(so.view(torch.int16).cpu().numpy().view(np.uint16).reshape(2, -1), ws)


def test_int4_integer_inputs_bit_exact():
    """Integer activations and unit scales: the result is an exact integer, so is its bf16."""
    require_gpu()
    rng = np.random.default_rng(9)
    E, N, K = 2, 256, 512
    counts = np.array([3, 11], np.int32)
    starts = np.array([0, 16, 32])
    ai = rng.integers(-3, 4, size=(32, K)).astype(np.float32)
    q = rng.integers(0, 16, size=(E, N, K)).astype(np.uint8)
    q4 = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    c = dict(E=E, N=N, K=K, rows=32, starts=starts, eff=counts, counts=counts, layout=moe.LAYOUT_MASKED, max_m=16,
             a=u16(torch.from_numpy(ai).to(torch.bfloat16)), q4=q4, s16=np.full((E, N, K // 128), 0x3C00, np.uint16))
    for em, packed in ((0, False), (16, False), (0, True), (16, True)):
        D = _run_int4(c, em, packed=packed)
        for e in range(E):
            s, n = int(starts[e]), int(counts[e])
            exact = ai[s:s + n].astype(np.int64) @ (q[e].astype(np.int64) - 8).T
            assert np.array_equal(u16(D)[s:s + n], oracle.f64_to_bf16_bits(exact.astype(np.float64)))


@pytest.mark.parametrize("packed", [False, True])
def test_int4_determinism_20_runs(packed):
    require_gpu()
    c = _int4_case(10, [4, 16, 0, 2], N=256, K=512, layout=moe.LAYOUT_MASKED, max_m=16)
    ref = _run_int4(c, packed=packed)
    for _ in range(20):
        assert torch.equal(_run_int4(c, packed=packed), ref)
