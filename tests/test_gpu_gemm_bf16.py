"""GPU BF16 grouped GEMM (moe_grouped_gemm_bf16) vs the oracle.

Bar (derived from the arithmetic): the GPU accumulates exact bf16 products in
fp32 and rounds the sum to bf16 once, so per element
  |D - y| <= 2^-8 |y| + 1e-5 * sum_k |a_k w_k|
(half a bf16 ulp of the fp32 result, plus a generous allowance for the fp32
accumulation), and calc_diff < 1e-5 (the pages' BF16 threshold, nxmr.cn
DeepGEMM article, "精度与吞吐的平衡点").  Small-integer inputs whose sums are
exact in bf16 must match bit for bit.
"""

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import oracle
import weight_layout as wl
from gpu_helpers import DEV, bf16_from_u16, require_gpu, u16

pytestmark = pytest.mark.gpu
SENT = 0x7BAD


def _layout(counts, layout, max_m=0, align=128):
    E = len(counts)
    if layout == moe.LAYOUT_MASKED:
        return np.arange(E + 1) * max_m, E * max_m, np.minimum(counts, max_m)
    starts = np.zeros(E + 1, np.int64)
    for e in range(E):
        starts[e + 1] = starts[e] + -(-counts[e] // align) * align
    return starts, max(int(starts[E]), align), np.array(counts)


def _case(seed, counts, N, K, layout, max_m=0, ints=False):
    rng = np.random.default_rng(seed)
    E = len(counts)
    starts, rows, eff = _layout(np.array(counts), layout, max_m)
    if ints:
        a = rng.integers(-1, 2, (rows, K)).astype(np.float32)
        w = rng.integers(-1, 2, (E, N, K)).astype(np.float32)
    else:
        a = rng.standard_normal((rows, K)).astype(np.float32)
        w = (rng.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    return dict(E=E, N=N, K=K, rows=rows, starts=starts, eff=eff, counts=np.array(counts, np.int32), layout=layout,
                max_m=max_m, a=oracle.f32_to_bf16_bits(a), w=oracle.f32_to_bf16_bits(w))


def _run(c, expected_m=0, packed=False):
    D = torch.full((c["rows"], c["N"]), SENT, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    am = c["max_m"] if c["layout"] == moe.LAYOUT_MASKED else c["rows"]
    if packed:
        w = bf16_from_u16(wl.pack_weight_bf16(c["w"]).reshape(c["w"].shape))
        layout = c["layout"] | moe.WEIGHTS_PACKED
    else:
        w, layout = bf16_from_u16(c["w"]), c["layout"]
    moe.moe_grouped_gemm_bf16(layout, bf16_from_u16(c["a"]), w, D,
                              torch.from_numpy(c["counts"]).to(DEV),
                              torch.from_numpy(c["starts"].astype(np.int32)).to(DEV), c["E"], am, c["N"], c["K"],
                              expected_m)
    torch.cuda.synchronize()
    return D


def _check(c, D, exact=False):
    ref = oracle.grouped_gemm_bf16(c["a"], c["w"], c["eff"], c["starts"])
    mag = oracle.grouped_gemm_bf16(oracle.f32_to_bf16_bits(np.abs(oracle.bf16_bits_to_f64(c["a"])).astype(np.float32)),
                                   oracle.f32_to_bf16_bits(np.abs(oracle.bf16_bits_to_f64(c["w"])).astype(np.float32)),
                                   c["eff"], c["starts"])
    valid = np.isfinite(ref[:, 0])
    bits = u16(D)
    assert (bits[~valid] == SENT).all(), "rows outside the segments were written"
    got = oracle.bf16_bits_to_f64(bits[valid])
    y, m = ref[valid], mag[valid]
    if exact:
        assert np.array_equal(got, y)
        return
    assert oracle.calc_diff(got, y) < 1e-5
    assert (np.abs(got - y) <= 2.0 ** -8 * np.abs(y) + 1e-5 * m).all()


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 16, 64, 128])
def test_bf16_contiguous_ragged(expected_m, packed):
    """expected_m picks the tile: 16 -> 16-row, 64 -> 64-row, 128 -> 192-row tall, 0 (= 256) -> 256-row tall."""
    require_gpu()
    c = _case(1, [0, 1, 17, 130, 300], N=384, K=1536, layout=moe.LAYOUT_CONTIGUOUS)
    _check(c, _run(c, expected_m, packed))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("expected_m", [0, 16])
def test_bf16_masked_clipped(expected_m, packed):
    require_gpu()
    c = _case(2, [5, 0, 64, 90, 1, 33], N=256, K=768, layout=moe.LAYOUT_MASKED, max_m=64)
    _check(c, _run(c, expected_m, packed))


@pytest.mark.parametrize("packed", [False, True])
def test_bf16_small_integers_bit_exact_and_deterministic(packed):
    require_gpu()
    c = _case(3, [7, 64, 129, 300], N=512, K=256, layout=moe.LAYOUT_CONTIGUOUS, ints=True)
    for em in (16, 64, 128, 256):
        D = _run(c, em, packed)
        _check(c, D, exact=True)
        for _ in range(10):
            assert torch.equal(_run(c, em, packed), D)


def test_bf16_many_experts_and_narrow_n():
    require_gpu()
    rng = np.random.default_rng(4)
    counts = rng.integers(0, 40, 300)
    c = _case(5, list(counts), N=128, K=256, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (0, 16, 64):
        _check(c, _run(c, em))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("K", [1536, 2560])
def test_bf16_tall_every_row_tile_count_long_k(K, packed):
    """Both tall heights on units of every 32-row count (1..256 rows, so every loop body), N = 384 (the second
    256-column tile has two idle waves), K/64 = 24 or 40 steps (main loop iterations before the last)."""
    require_gpu()
    counts = [32 * r - 5 for r in range(1, 9)] + [32 * r for r in range(1, 9)] + [0, 3, 256 + 100, 192 + 40]
    c = _case(61 + K, counts, N=384, K=K, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (128, 256):
        _check(c, _run(c, em, packed))


@pytest.mark.parametrize("packed", [False, True])
def test_bf16_tall_masked_segments_and_short_k_fallback(packed):
    """Masked segments taller than a tall tile, and K/64 not a multiple of 4 (the tall loop cannot run: the
    64-row tile takes prefill-sized calls)."""
    require_gpu()
    c = _case(12, [150, 0, 300, 65], N=256, K=1024, layout=moe.LAYOUT_MASKED, max_m=300)
    for em in (0, 200, 256):
        _check(c, _run(c, em, packed))
    c = _case(14, [0, 1, 17, 130, 300], N=256, K=384, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (0, 128):
        _check(c, _run(c, em, packed))


@pytest.mark.parametrize("packed", [False, True])
def test_bf16_degenerate_expert_counts(packed):
    """No rows at all, 1024 experts with 0..3 rows (N = 128: half of each tall tile's waves store nothing), and
    one expert with several tall chunks, on every tile height."""
    require_gpu()
    c = _case(31, [0] * 8, N=256, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (16, 64, 128, 256):
        _check(c, _run(c, em, packed))
    counts = np.random.default_rng(33).integers(0, 4, size=1024).tolist()
    c = _case(33, counts, N=128, K=256, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (16, 128, 256):
        _check(c, _run(c, em, packed))
    c = _case(34, [700], N=384, K=512, layout=moe.LAYOUT_CONTIGUOUS)
    for em in (64, 128, 256):
        _check(c, _run(c, em, packed))


def test_pack_weight_bf16_bit_exact():
    require_gpu()
    rng = np.random.default_rng(9)
    E, N, K = 3, 384, 640
    w = rng.integers(0, 1 << 16, size=(E, N, K), dtype=np.uint16)
    out = torch.zeros(E, N, K, dtype=torch.bfloat16, device=DEV)
    moe.moe_pack_weight_bf16(bf16_from_u16(w), out)
    torch.cuda.synchronize()
    assert np.array_equal(u16(out).reshape(E, N * K), wl.pack_weight_bf16(w))


def test_bf16_full_size_dsv3_decode_and_prefill_samples():
    """DeepSeek-V3-shaped experts (K=7168, N=4096) with bf16 weights: every route's rows of sampled experts, at
    three 128-column blocks, for the decode (masked, 64 rows) and prefill (contiguous) routings."""
    require_gpu()
    import synth

    for name in ("dsv3_decode", "dsv3_prefill"):
        cfg = synth.config_by_name(name)
        print(f"[bf16] {name}", flush=True)
        ids, _ = synth.route_inputs(cfg)
        E, K, N = cfg.E, cfg.K, cfg.N
        layout = moe.LAYOUT_MASKED if cfg.layout == "masked" else moe.LAYOUT_CONTIGUOUS
        am = cfg.max_m if cfg.layout == "masked" else cfg.align
        lay = "masked" if cfg.layout == "masked" else "contiguous"
        kw = {"max_m": am} if lay == "masked" else {"align": am}
        r = oracle.route(ids.numpy(), E, lay, **kw)
        rows = r["rows_cap"]
        # packed rows of seeded activations; expert weights drawn on the GPU (bf16)
        A = synth.activations(cfg, rows, K, device=DEV)
        W = torch.empty(E, N, K, dtype=torch.bfloat16, device=DEV)
        for e0 in range(0, E, 32):
            W[e0:e0 + 32] = synth.expert_weights(cfg, N, K, experts=range(e0, min(E, e0 + 32)), device=DEV)
        D = torch.full((rows, N), SENT, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        em = max(1, cfg.T * cfg.topk // E)
        moe.moe_grouped_gemm_bf16(layout, A, W, D, torch.from_numpy(r["counts"].astype(np.int32)).to(DEV),
                                  torch.from_numpy(r["seg_offsets"].astype(np.int32)).to(DEV), E,
                                  cfg.max_m if lay == "masked" else rows, N, K, em)
        torch.cuda.synchronize()
        counts = r["counts"]
        active = np.nonzero(counts)[0]
        sample = sorted({int(active[np.argmax(counts[active])]), int(active[np.argmin(counts[active])]),
                         int(active[len(active) // 2])})
        blocks = [0, 13, N // 128 - 1]
        cols = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
        for e in sample:
            st, cnt = int(r["seg_offsets"][e]), int(counts[e])
            sel = torch.arange(st, st + cnt, device=DEV)
            a = u16(A[sel])
            w = u16(W[e][torch.from_numpy(cols).to(DEV)])[None]
            c = dict(a=a, w=w, eff=np.array([cnt]), starts=np.array([0, cnt]))
            ref = oracle.grouped_gemm_bf16(a, w, c["eff"], c["starts"])
            got = oracle.bf16_bits_to_f64(u16(D[sel][:, torch.from_numpy(cols).to(DEV)]))
            mag = np.abs(oracle.bf16_bits_to_f64(a)) @ np.abs(oracle.bf16_bits_to_f64(w[0])).T
            assert oracle.calc_diff(got, ref) < 1e-5
            assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * mag).all()
        # padding rows of the segments stay untouched
        e = sample[0]
        st, cnt = int(r["seg_offsets"][e]), int(counts[e])
        end = st + (am if lay == "masked" else -(-cnt // am) * am)
        if end > st + cnt:
            assert (u16(D[st + cnt:end]) == SENT).all()
        del W, D, A
        torch.cuda.empty_cache()
