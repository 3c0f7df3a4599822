"""GPU MXFP4 weight quantiser and FP8 x FP4 grouped GEMM vs the oracle.

Quantisation is bit-exact (power-of-two scales, exact multiplies, RNE).  The
GEMM is compared with the oracle's exact sum on the same quantised operands:
calc_diff < 1e-3 and |D - y| <= 2e-2 |y| + 1e-2 rms(y) (the FP8 GEMM's bar; the
pages' 0.01 for one FP4 side measures the quantisation itself, against
unquantised inputs, which is reported separately).  Where the exact result is
representable the GPU must match it bit for bit: one-hot activation rows
(which also pin how K, the nibble order and the 32-value scale blocks line up
between the two operand formats) and small integers.
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


def _quant_w_gpu(w_bits):
    E, N, K = w_bits.shape
    w4 = torch.empty(E, N, K // 2, dtype=torch.uint8, device=DEV)
    sw = torch.empty(E, N, K // 32, dtype=torch.uint8, device=DEV)
    moe.moe_quant_weight_fp4(bf16_from_u16(w_bits.reshape(E * N, K)).view(E, N, K), w4, sw)
    torch.cuda.synchronize()
    return w4.cpu().numpy(), sw.cpu().numpy()


def test_quant_weight_fp4_bit_exact():
    require_gpu()
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((3, 128, 512)) * 0.02).astype(np.float32)
    w[0, 0, :32] = 0.0                       # an all-zero block: scale byte 127, zero codes
    w[0, 1, 32:64] *= 1e6                    # large values
    w[1, 2, :] *= 1e-30                      # tiny values
    w[2, 3, 5] = -1e-45                      # rounds to -0 within its block
    w[2, 4, :32] = np.float32(6.0) * np.arange(32) / 31  # values up to exactly 6 * 2^0
    bits = oracle.f32_to_bf16_bits(w)
    g4, gs = _quant_w_gpu(bits)
    o4, os_ = oracle.quant_weight_fp4(bits)
    assert np.array_equal(gs, os_) and np.array_equal(g4, o4)


def _case(seed, counts, N, K, layout, max_m=0, ints=False):
    rng = np.random.default_rng(seed)
    E = len(counts)
    if layout == moe.LAYOUT_MASKED:
        starts, rows, eff = np.arange(E + 1) * max_m, E * max_m, np.minimum(counts, max_m)
    else:
        starts = np.zeros(E + 1, np.int64)
        for e in range(E):
            starts[e + 1] = starts[e] + -(-counts[e] // 128) * 128
        rows, eff = max(int(starts[E]), 128), np.array(counts)
    if ints:
        ints8 = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44}
        ai = rng.integers(-3, 4, (rows, K))
        a = np.vectorize(lambda v: ints8[abs(v)] | (0x80 if v < 0 else 0))(ai).astype(np.uint8)
        sa = np.ones((rows, K // 128), np.float32)
        wv = rng.choice([-6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6], size=(E, N, K)).astype(np.float64)
        q = oracle.e2m1_encode(wv)
        w4 = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
        sw = np.full((E, N, K // 32), 127, np.uint8)
    else:
        x = rng.standard_normal((rows, K)).astype(np.float32)
        a, sa = oracle.quant_act(oracle.f32_to_bf16_bits(x))
        w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
        w4, sw = oracle.quant_weight_fp4(oracle.f32_to_bf16_bits(w))
    return dict(E=E, N=N, K=K, rows=rows, starts=starts, eff=eff, counts=np.array(counts, np.int32), layout=layout,
                max_m=max_m, a=a, sa=sa, w4=w4, sw=sw)


def _run(c, expected_m=0, packed=False):
    """packed: the weights go in the test helper's packed order with MOE_WEIGHTS_PACKED."""
    D = torch.full((c["rows"], c["N"]), SENT, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    am = c["max_m"] if c["layout"] == moe.LAYOUT_MASKED else c["rows"]
    w4, sw = c["w4"], c["sw"]
    if packed:
        w4, sw = wl.pack_weight_fp4(w4, sw)
        w4, sw = w4.reshape(c["w4"].shape), sw.reshape(c["sw"].shape)
    layout = c["layout"] | (moe.WEIGHTS_PACKED if packed else 0)
    moe.moe_grouped_gemm_fp8_fp4(layout, torch.from_numpy(c["a"]).to(DEV), torch.from_numpy(c["sa"]).to(DEV),
                                 torch.from_numpy(np.ascontiguousarray(w4)).to(DEV),
                                 torch.from_numpy(np.ascontiguousarray(sw)).to(DEV), D,
                                 torch.from_numpy(c["counts"]).to(DEV),
                                 torch.from_numpy(c["starts"].astype(np.int32)).to(DEV), c["E"], am, c["N"], c["K"],
                                 expected_m)
    torch.cuda.synchronize()
    return D


def _ref(c):
    return oracle.grouped_gemm_fp8_fp4(c["a"], c["sa"], c["w4"], c["sw"], c["eff"], c["starts"])


def _check(c, D, exact=False):
    ref = _ref(c)
    valid = np.isfinite(ref[:, 0])
    bits = u16(D)
    assert (bits[~valid] == SENT).all(), "rows outside the segments were written"
    if exact:
        want = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits_normal(ref[valid]))
        assert np.array_equal(oracle.bf16_bits_to_f64(bits[valid]), want)
        return
    gemm_tolerance_check(oracle.bf16_bits_to_f64(bits[valid]), ref[valid], 1e-3)


@pytest.mark.parametrize("packed,expected_m", [(False, 64), (True, 64), (True, 128), (True, 256)])
def test_fp4_one_hot_rows_pin_the_operand_layout(packed, expected_m):
    """Row r has one activation 2.0 at k_r (scale 1): D[r] = 2 * column k_r of the dequantised weights, exactly
    (packed: also pins which byte of the scale dword each step's instruction selects; expected_m 128 and 256 run
    the tall tiles, whose 32x32x64 instruction lays K out differently from the 16x16x128 one)."""
    require_gpu()
    c = _case(2, [40], N=256, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    ks = [0, 1, 2, 31, 32, 33, 63, 64, 95, 127, 128, 129, 200, 255, 300, 383, 384, 447, 510, 511] + list(range(3, 23))
    c["a"][:] = 0
    c["sa"][:] = 1.0
    for r, k in enumerate(ks[:40]):
        c["a"][r, k] = 0x40
    D = _run(c, expected_m, packed)
    bits = u16(D)[:40]
    wd = oracle.dequant_weight_fp4(c["w4"][0], c["sw"][0])
    for r, k in enumerate(ks[:40]):
        # values, not bit patterns: the fp32 accumulator starts at +0, so a zero column sums to +0 where the
        # oracle's single product is -0
        want = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits_normal(2.0 * wd[:, k]))
        assert np.array_equal(oracle.bf16_bits_to_f64(bits[r]), want), f"row {r}, k {k}"


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 16, 64])
def test_fp4_contiguous_ragged(expected_m, packed):
    require_gpu()
    c = _case(3, [0, 1, 17, 130, 300], N=384, K=1536, layout=moe.LAYOUT_CONTIGUOUS)
    _check(c, _run(c, expected_m, packed))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 16])
def test_fp4_masked_clipped(expected_m, packed):
    require_gpu()
    c = _case(4, [5, 0, 64, 90, 1, 33], N=256, K=768, layout=moe.LAYOUT_MASKED, max_m=64)
    _check(c, _run(c, expected_m, packed))


def test_pack_weight_fp4_matches_the_layout_definition():
    require_gpu()
    rng = np.random.default_rng(8)
    E, N, K = 3, 256, 896
    w4 = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    sw = rng.integers(0, 255, (E, N, K // 32), dtype=np.uint8)
    w4p = torch.empty(E, N, K // 2, dtype=torch.uint8, device=DEV)
    swp = torch.empty(E, N, K // 32, dtype=torch.uint8, device=DEV)
    moe.moe_pack_weight_fp4(torch.from_numpy(w4).to(DEV), torch.from_numpy(sw).to(DEV), w4p, swp)
    torch.cuda.synchronize()
    cw, cs = wl.pack_weight_fp4(w4, sw)
    assert np.array_equal(w4p.cpu().numpy().reshape(E, -1), cw)
    assert np.array_equal(swp.cpu().numpy().reshape(E, -1), cs)


@pytest.mark.parametrize("packed,expected_m", [(False, 64), (True, 64), (True, 128), (True, 256)])
def test_fp4_small_integers_exact_and_deterministic(packed, expected_m):
    require_gpu()
    c = _case(5, [7, 64, 129, 300], N=512, K=512, layout=moe.LAYOUT_CONTIGUOUS, ints=True)
    D = _run(c, expected_m, packed)
    _check(c, D, exact=True)
    for _ in range(20):
        assert torch.equal(_run(c, expected_m, packed), D)


@pytest.mark.parametrize("K", [1536, 2560])
def test_fp4_tall_every_row_tile_count_long_k(K):
    """Packed weights on both tall heights: units of every 32-row count (1..256 rows, so every loop body),
    N = 384 (the second 256-column tile has two idle waves), K/128 = 12 or 20 blocks (main loop iterations
    before the last)."""
    require_gpu()
    counts = [32 * r - 5 for r in range(1, 9)] + [32 * r for r in range(1, 9)] + [0, 3, 256 + 100, 192 + 40]
    c = _case(71 + K, counts, N=384, K=K, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (128, 256):
        _check(c, _run(c, em, True))


def test_fp4_tall_masked_segments_and_short_k_fallback():
    """Masked segments taller than a tall tile; K/128 not a multiple of 4 (the tall loop's row-scale copies
    cover 4 K blocks: such calls run on the 64-row tile)."""
    require_gpu()
    c = _case(12, [150, 0, 300, 65], N=256, K=1024, layout=moe.LAYOUT_MASKED, max_m=300)
    for em in (0, 200, 256):
        _check(c, _run(c, em, True))
    c = _case(14, [0, 1, 17, 130, 300], N=256, K=640, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (0, 128, 256):
        _check(c, _run(c, em, True))


def test_fp4_tall_degenerate_expert_counts():
    """No rows at all, 1024 experts with 0..3 rows (N = 128: half of each tall tile's waves store nothing), and
    one expert with several tall chunks."""
    require_gpu()
    c = _case(31, [0] * 8, N=256, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (128, 256):
        _check(c, _run(c, em, True))
    counts = np.random.default_rng(33).integers(0, 4, size=1024).tolist()
    c = _case(33, counts, N=128, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (128, 256):
        _check(c, _run(c, em, True))
    c = _case(34, [700], N=384, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (128, 256):
        _check(c, _run(c, em, True))


def test_fp4_full_size_dsv3_decode_and_prefill_samples():
    """DeepSeek-V3-shaped experts (K=7168, N=4096) with MXFP4 weights quantised on the GPU (checked bit-exactly
    on the sampled experts), the decode (masked, 64 rows) and prefill (contiguous) routings, sampled outputs;
    plus the quantisation error of the FP8 x FP4 product against the unquantised inputs (the pages' 0.01)."""
    require_gpu()
    import synth

    for name in ("dsv3_decode", "dsv3_prefill"):
        cfg = synth.config_by_name(name)
        print(f"[fp4] {name}", flush=True)
        ids, _ = synth.route_inputs(cfg)
        E, K, N = cfg.E, cfg.K, cfg.N
        lay = "masked" if cfg.layout == "masked" else "contiguous"
        am = cfg.max_m if lay == "masked" else cfg.align
        r = oracle.route(ids.numpy(), E, lay, **({"max_m": am} if lay == "masked" else {"align": am}))
        rows = r["rows_cap"]
        x = synth.activations(cfg, rows, K, device=DEV)
        A = torch.empty(rows, K, dtype=torch.uint8, device=DEV)
        SFA = torch.empty(rows, K // 128, dtype=torch.float32, device=DEV)
        moe.moe_quant_act(x, A, SFA)
        W4 = torch.empty(E, N, K // 2, dtype=torch.uint8, device=DEV)
        SW = torch.empty(E, N, K // 32, dtype=torch.uint8, device=DEV)
        counts = r["counts"]
        active = np.nonzero(counts)[0]
        sample = sorted({int(active[np.argmax(counts[active])]), int(active[np.argmin(counts[active])]),
                         int(active[len(active) // 2])})
        kept = {}
        for e0 in range(0, E, 32):
            ex = list(range(e0, min(E, e0 + 32)))
            w = synth.expert_weights(cfg, N, K, experts=ex, device=DEV)
            moe.moe_quant_weight_fp4(w, W4[e0:e0 + len(ex)], SW[e0:e0 + len(ex)])
            for i, e in enumerate(ex):
                if e in sample:
                    kept[e] = u16(w[i])
            del w
        D = torch.full((rows, N), SENT, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        W4p, SWp = torch.empty_like(W4), torch.empty_like(SW)
        moe.moe_pack_weight_fp4(W4, SW, W4p, SWp)  # the benchmark's weight order
        moe.moe_grouped_gemm_fp8_fp4((moe.LAYOUT_MASKED if lay == "masked" else moe.LAYOUT_CONTIGUOUS) |
                                     moe.WEIGHTS_PACKED, A, SFA, W4p, SWp,
                                     D, torch.from_numpy(counts.astype(np.int32)).to(DEV),
                                     torch.from_numpy(r["seg_offsets"].astype(np.int32)).to(DEV), E,
                                     am if lay == "masked" else rows, N, K, max(1, cfg.T * cfg.topk // E))
        torch.cuda.synchronize()
        blocks = [0, 13, N // 128 - 1]
        cols = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
        colsel = torch.from_numpy(cols).to(DEV)
        for e in sample:
            st, cnt = int(r["seg_offsets"][e]), int(counts[e])
            sel = torch.arange(st, st + cnt, device=DEV)
            a_c, a_s = oracle.quant_act(u16(x[sel]))
            assert np.array_equal(A[sel].cpu().numpy(), a_c)
            wq, ws = oracle.quant_weight_fp4(kept[e][cols][None])
            assert np.array_equal(W4[e][colsel].cpu().numpy(), wq[0]) and np.array_equal(SW[e][colsel].cpu().numpy(), ws[0])
            ref = oracle.dequant_act(a_c, a_s) @ oracle.dequant_weight_fp4(wq[0], ws[0]).T
            got = oracle.bf16_bits_to_f64(u16(D[sel][:, colsel]))
            gemm_tolerance_check(got, ref, 1e-3)
            # the FP8 x FP4 product against the unquantised bf16 inputs: the pages' one-FP4-side bar
            raw = oracle.bf16_bits_to_f64(u16(x[sel])) @ oracle.bf16_bits_to_f64(kept[e][cols]).T
            assert oracle.calc_diff(got, raw) < 1e-2
        del W4, SW, W4p, SWp, D, A, x
        torch.cuda.empty_cache()
