"""Full-size parity: every workload at its measured shape, launched the way the
benchmark launches it (MoeFP8Layer / MoeInt4Layer, tiling hint = routes per
expert; for the FP8 workloads both the two-call quantise + pack and the
quantising pack the benchmark times), checked against the oracle.

Routing and packing are checked bit-exactly on every route; activation and
weight quantisation bit-exactly on sampled token rows and weight blocks; the
grouped GEMM and the combine on sampled outputs the oracle can compute one by
one: the rows of a few experts (the most and least loaded, and every expert of
one sampled token), at three 128-column blocks of N chosen so that they fall in
different waves of different N tiles.  The oracle never sees a value produced
by the HIP path: its activations and weights are the seeded bf16 inputs, copied
to the host and quantised by the oracle itself.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import oracle
import synth
from gpu_helpers import DEV, gemm_tolerance_check, require_gpu, u16
from int4_weights_amd.layer import MoeFP8Layer, MoeInt4Layer

pytestmark = pytest.mark.gpu


def _sample_experts(ids: np.ndarray, E: int, tok: int):
    counts = np.bincount(ids.reshape(-1), minlength=E)
    active = np.nonzero(counts)[0]
    top = int(active[np.argmax(counts[active])])
    low = int(active[np.argmin(counts[active])])
    return sorted(set([top, low] + [int(e) for e in ids[tok]])), counts


def _col_blocks(N: int):
    nb = N // 128
    return sorted(set([0, min(3, nb - 1), nb - 1]))


def _rows_of(start: int, count: int, cap: int = 200):
    """Packed rows of a segment: all of them, or the edges and the 192/256-row tile seams of a long one."""
    if count <= cap:
        return np.arange(start, start + count)
    pick = set(range(0, 40)) | set(range(count - 40, count))
    for seam in (128, 192, 256, 384, 512):
        for m in range(seam, count, seam * 7):
            pick |= set(range(max(0, m - 3), min(count, m + 3)))
    return start + np.array(sorted(pick))


def _gpu_fp8_weights(cfg, N, K, stream, keep):
    """Expert weights drawn on the GPU, quantised by the library (row-major codes, checked against the
    oracle) and packed by the library into the order the benchmark's layer reads; bf16 copies of
    `keep` on the host."""
    E = cfg.E
    codes = torch.empty(E, N, K, dtype=torch.uint8, device=DEV)
    packed = torch.empty(E, N, K, dtype=torch.uint8, device=DEV)
    sfw = torch.empty(E, N // 128, K // 128, dtype=torch.float32, device=DEV)
    kept = {}
    for e0 in range(0, E, 16):
        ex = list(range(e0, min(E, e0 + 16)))
        w = synth.expert_weights(cfg, N, K, experts=ex, stream=stream, device=DEV)
        moe.moe_quant_weight_fp8(w, codes[e0:e0 + len(ex)], sfw[e0:e0 + len(ex)])
        for i, e in enumerate(ex):
            if e in keep:
                kept[e] = u16(w[i])
        del w
    moe.moe_pack_weight_fp8(codes, packed)
    torch.cuda.synchronize()
    return codes, sfw, kept, packed


def _check_routing(layer, ids_np, E, layout_name, am):
    kw = {"align": am} if layout_name == "contiguous" else {"max_m": am}
    rows = layer.rows_cap
    if layout_name == "contiguous":
        rows = moe.moe_packed_rows_cap(ids_np.shape[0], ids_np.shape[1], E, am)
    r = oracle.route(ids_np, E, layout_name, rows_cap=rows, **kw)
    T = ids_np.shape[0]
    assert np.array_equal(layer.counts.cpu().numpy(), r["counts"])
    assert np.array_equal(layer.seg_offsets.cpu().numpy(), r["seg_offsets"])
    assert np.array_equal(layer.output_index[:T].cpu().numpy(), r["output_index"])
    assert np.array_equal(layer.m_indices[:rows].cpu().numpy(), r["m_indices"])
    assert int(layer.dev_status.item()) == r["status"]
    return r


def _token_of_rows(r, T):
    """packed row -> (token, slot) from the oracle's routing."""
    oi = r["output_index"]
    owner = {}
    for t in range(T):
        for s in range(oi.shape[1]):
            if oi[t, s] >= 0:
                owner[int(oi[t, s])] = (t, s)
    return owner


def _fp8_layer_case(cfg, seed_tok):
    T, E, k, K, N = cfg.T, cfg.E, cfg.topk, cfg.K, cfg.N
    ids, tw = synth.route_inputs(cfg)
    ids_np = ids.numpy()
    tok = seed_tok % T
    sample, counts = _sample_experts(ids_np, E, tok)
    x = synth.activations(cfg, T, K)
    codes, sfw, kept, packed = _gpu_fp8_weights(cfg, N, K, synth.STREAM_WEIGHTS, set(sample))
    layout = moe.LAYOUT_MASKED if cfg.layout == "masked" else moe.LAYOUT_CONTIGUOUS
    am = cfg.max_m if cfg.layout == "masked" else cfg.align
    layer = MoeFP8Layer(packed, sfw, k, T, layout, am, expected_m=max(1, T * k // E), weights_packed=True)
    z = layer.forward(x.to(DEV), ids.to(DEV), tw.to(DEV))
    torch.cuda.synchronize()
    return dict(T=T, E=E, k=k, K=K, N=N, ids=ids_np, tw=tw.numpy(), tok=tok, sample=sample, x=x, codes=codes,
                sfw=sfw, kept=kept, layer=layer, z=z, am=am, packed=packed)


def _check_quant_rows(layer, x_bits, tokens):
    a_c, a_s = oracle.quant_act(x_bits[tokens])
    assert np.array_equal(layer.q[tokens].cpu().numpy(), a_c)
    assert np.array_equal(layer.sf[tokens].cpu().numpy(), a_s)


def _check_packing(layer, r, T):
    """Every valid route's packed row equals its token's quantised row (bytes and scale row)."""
    oi = r["output_index"].reshape(-1)
    ok = oi >= 0
    tok = (np.arange(oi.size) // r["output_index"].shape[1])[ok]
    rows = torch.from_numpy(oi[ok].astype(np.int64)).to(DEV)
    src = torch.from_numpy(tok.astype(np.int64)).to(DEV)
    assert torch.equal(layer.packed[rows], layer.q[:T][src])
    assert torch.equal(layer.packed_sf[rows], layer.sf[:T][src])


def _fp8_gemm_and_combine(c, r, A_bits_of_token, D, Z, kept_codes_fn, label):
    """Oracle GEMM on sampled rows x sampled column blocks, then the combine of the sampled token."""
    N, K = c["N"], c["K"]
    blocks = _col_blocks(N)
    cols = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
    owner = _token_of_rows(r, c["T"])
    y_ref_rows = {}
    for e in c["sample"]:
        cnt, st = int(r["counts"][e]), int(r["seg_offsets"][e])
        if cnt == 0:
            continue
        rows = list(_rows_of(st, cnt))
        # the sampled token's route into e is always among the rows
        for s in range(c["k"]):
            p = int(r["output_index"][c["tok"], s])
            if p >= st and p < st + cnt and p not in rows:
                rows.append(p)
        rows = np.array(sorted(rows))
        toks = np.array([owner[int(p)][0] for p in rows])
        w_sub = kept_codes_fn(e, blocks)  # float64 [len(cols), K] (oracle-quantised)
        y = A_bits_of_token(toks) @ w_sub.T
        got = D[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].float().cpu().numpy()
        gemm_tolerance_check(got.astype(np.float64), y, 1e-3 if label == "fp8" else 1e-2)
        for i, p in enumerate(rows):
            y_ref_rows[int(p)] = y[i]
    # combine of the sampled token over the sampled columns
    t = c["tok"]
    zr = np.zeros(len(cols))
    for s in range(c["k"]):
        p = int(r["output_index"][t, s])
        if p >= 0:
            zr += float(c["tw"][t, s]) * y_ref_rows[p]
    zg = Z[t][torch.from_numpy(cols).to(DEV)].float().cpu().numpy().astype(np.float64)
    gemm_tolerance_check(zg[None], zr[None], 1e-3 if label == "fp8" else 1e-2)


def _check_fused_quant_pack(layer, x, ids, r, T):
    """The benchmark's launch: moe_route_pack_quant (quantise while packing) gives the same routing outputs and
    the same packed codes and scale rows, on every valid route, as the two-call path checked against the oracle."""
    oiv = r["output_index"].reshape(-1)
    rows = torch.from_numpy(oiv[oiv >= 0].astype(np.int64)).to(DEV)
    pk, psf = layer.packed[rows].clone(), layer.packed_sf[rows].clone()
    mi, oi = layer.m_indices.clone(), layer.output_index[:T].clone()
    layer.packed[rows] = 0
    layer.packed_sf[rows] = -1.0
    layer.quant_route(x.to(DEV), ids.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(layer.packed[rows], pk)
    assert torch.equal(layer.packed_sf[rows].view(torch.int32), psf.view(torch.int32))
    assert torch.equal(layer.m_indices, mi) and torch.equal(layer.output_index[:T], oi)


def _oracle_fp8_weight_blocks(c, codes, sfw, kept, N, K):
    """Oracle quantisation of the sampled 128-row blocks of an expert, checked bit-exactly against the GPU's."""
    cache = {}

    def fn(e, blocks):
        if e not in cache:
            wb = kept[e]
            sub = np.concatenate([wb[128 * b:128 * b + 128] for b in blocks])[None]
            q, s = oracle.quant_weight_fp8(sub)
            rows = torch.from_numpy(np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])).to(DEV)
            assert np.array_equal(codes[e][rows].cpu().numpy(), q[0]), f"weight codes of expert {e}"
            assert np.array_equal(sfw[e][torch.tensor(blocks, device=DEV)].cpu().numpy(), s[0]), f"sfw of {e}"
            cache[e] = oracle.dequant_weight_fp8(q[0], s[0])
        return cache[e]

    return fn


@pytest.mark.parametrize("name", ["tiny", "dsv3_prefill", "dsv3_decode"])
def test_full_size_fp8_layer(name):
    require_gpu()
    cfg = synth.config_by_name(name)
    print(f"[fullsize] {name}", flush=True)
    c = _fp8_layer_case(cfg, seed_tok=cfg.T // 2 + 1)
    layer = c["layer"]
    r = _check_routing(layer, c["ids"], c["E"], cfg.layout, c["am"])
    x_bits = u16(c["x"])
    toks = sorted(set([0, c["T"] - 1, c["tok"]] + list(range(1, c["T"], max(1, c["T"] // 16)))))
    _check_quant_rows(layer, x_bits, np.array(toks))
    _check_packing(layer, r, c["T"])
    _check_fused_quant_pack(layer, c["x"], torch.from_numpy(c["ids"]), r, c["T"])

    def a_of_tokens(tt):
        a, sa = oracle.quant_act(x_bits[tt])
        return oracle.dequant_act(a, sa)

    fn = _oracle_fp8_weight_blocks(c, c["codes"], c["sfw"], c["kept"], c["N"], c["K"])
    _fp8_gemm_and_combine(c, r, a_of_tokens, layer.D, c["z"], fn, "fp8")


def test_full_size_qwen3_skewed_up_down_combine():
    """Zipf-skewed prefill: up-projection, SwiGLU + requantisation, down-projection, combine of the down output."""
    require_gpu()
    cfg = synth.config_by_name("qwen3_skewed")
    print("[fullsize] qwen3_skewed", flush=True)
    c = _fp8_layer_case(cfg, seed_tok=4097)
    layer = c["layer"]
    r = _check_routing(layer, c["ids"], c["E"], "contiguous", c["am"])
    x_bits = u16(c["x"])
    _check_quant_rows(layer, x_bits, np.array([0, 1, c["tok"], c["T"] - 1]))
    _check_packing(layer, r, c["T"])
    _check_fused_quant_pack(layer, c["x"], torch.from_numpy(c["ids"]), r, c["T"])

    def a_of_tokens(tt):
        a, sa = oracle.quant_act(x_bits[tt])
        return oracle.dequant_act(a, sa)

    fn = _oracle_fp8_weight_blocks(c, c["codes"], c["sfw"], c["kept"], c["N"], c["K"])
    _fp8_gemm_and_combine(c, r, a_of_tokens, layer.D, c["z"], fn, "fp8")
    del c["codes"], c["packed"]

    # down-projection on SwiGLU(gate, up) of the up-projection's output, requantised by moe_swiglu_quant, as the
    # layer runs it (the up-projection's 3072 columns are gate 0..1535 and up 1536..3071)
    Kd, Nd = cfg.K_down, cfg.N_down
    assert c["N"] == 2 * Kd
    dcodes, dsfw, dkept, dpacked = _gpu_fp8_weights(cfg, Nd, Kd, synth.STREAM_WEIGHTS_DOWN, set(c["sample"]))
    qd = torch.empty(layer.rows_cap, Kd, dtype=torch.uint8, device=DEV)
    sfd = torch.empty(layer.rows_cap, Kd // 128, dtype=torch.float32, device=DEV)
    Dd = torch.empty(layer.rows_cap, Nd, dtype=torch.bfloat16, device=DEV)
    Zd = torch.empty(c["T"], Nd, dtype=torch.bfloat16, device=DEV)
    layer.swiglu_quant(qd, sfd)
    # the up-projection with SwiGLU fused gives the same bits on every valid row (checked below against the
    # oracle through qd on the sampled rows)
    qf = torch.full((layer.rows_cap, Kd), 0xA5, dtype=torch.uint8, device=DEV)
    sff = torch.full((layer.rows_cap, Kd // 128), -3.0, dtype=torch.float32, device=DEV)
    print("[fullsize] qwen3_skewed fused up-projection + SwiGLU", flush=True)
    layer.gemm_swiglu(qf, sff)
    layer.gemm(A=qd, SFA=sfd, D=Dd, w=dpacked, sfw=dsfw, N=Nd, K=Kd)
    layer.combine(torch.from_numpy(c["tw"]).to(DEV), D=Dd, Z=Zd)
    torch.cuda.synchronize()

    # The oracle chain, by the path's definitions: the up-projection's exact output rounded to bf16 (the GEMM's
    # output format), SwiGLU and the 1x128 requantisation of those values, the down-projection in float64.
    owner = _token_of_rows(r, c["T"])
    fnd = _oracle_fp8_weight_blocks(c, dcodes, dsfw, dkept, Nd, Kd)
    blocks = _col_blocks(Nd)
    cols = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
    yrow = {}
    flips = total = 0
    for e in c["sample"]:
        cnt, st = int(r["counts"][e]), int(r["seg_offsets"][e])
        if cnt == 0:
            continue
        rows = set(_rows_of(st, cnt).tolist())
        rows |= set(int(p) for p in r["output_index"][c["tok"]] if st <= p < st + cnt)
        rows = np.array(sorted(rows))
        toks = np.array([owner[int(p)][0] for p in rows])
        wq, ws = oracle.quant_weight_fp8(c["kept"][e][None])
        y_up = a_of_tokens(toks) @ oracle.dequant_weight_fp8(wq[0], ws[0]).T
        qo, so = oracle.swiglu_quant(oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits_normal(y_up)))
        sel = torch.from_numpy(rows).to(DEV)
        qg = qd[sel].cpu().numpy()
        flips += int((qg != qo).sum())
        total += qo.size
        wd = fnd(e, blocks)
        y = oracle.dequant_act(qo, so) @ wd.T
        got = Dd[sel][:, torch.from_numpy(cols).to(DEV)].float().cpu().numpy().astype(np.float64)
        _chain_check(got, y, qo, so, wd)
        for i, p in enumerate(rows):
            yrow[int(p)] = y[i]
    # codes differ only where the GPU's up-projection rounds to another bf16 than the exact value (the FP8 matrix
    # instruction's accumulation, about 1% of its outputs by one ulp) or the fp32 SwiGLU lands on the other side of
    # an E4M3 rounding midpoint: rare
    assert flips <= total // 200, f"{flips} of {total} SwiGLU codes differ"
    vrows = np.zeros(layer.rows_cap, bool)
    for e in range(c["E"]):
        st = int(r["seg_offsets"][e])
        vrows[st:st + int(r["counts"][e])] = True
    vsel = torch.from_numpy(vrows).to(DEV)
    assert torch.equal(qf[vsel], qd[vsel]) and torch.equal(sff[vsel], sfd[vsel])
    assert (qf[~vsel] == 0xA5).all() and (sff[~vsel] == -3.0).all()
    t = c["tok"]
    zr = sum(float(c["tw"][t, s]) * yrow[int(r["output_index"][t, s])] for s in range(c["k"]))
    zg = Zd[t][torch.from_numpy(cols).to(DEV)].float().cpu().numpy().astype(np.float64)
    assert oracle.calc_diff(zg, zr) < 1e-3


def _chain_check(got, y, qo, so, wd):
    """Down-projection output after the GPU's own up-projection and SwiGLU vs the oracle chain.

    The requantised codes of the two chains can differ by one E4M3 step where the up-projection's bf16 output
    differs from the exact rounding (see the flip count).  The bar: the pages' calc_diff < 1e-3; every element
    within the GEMM bound 2e-2*|y| + 1e-2*rms(y) plus three such steps at the element's largest |step * w|; and
    99.5% of the elements within the GEMM bound alone."""
    assert oracle.calc_diff(got, y) < 1e-3
    tab = oracle.e4m3_decode_table()
    v = np.abs(tab[qo])
    # one E4M3 step at each code's magnitude (2^-9 in the subnormal range), times the block scale
    step = np.where(v < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3))
    step = step * np.repeat(so.astype(np.float64), 128, axis=1)
    aw = np.abs(wd)
    worst = np.concatenate([np.max(step[i:i + 8, None, :] * aw[None], axis=2) for i in range(0, len(step), 8)])
    rms = float(np.sqrt(np.mean(y * y)))
    bound = 2e-2 * np.abs(y) + 1e-2 * rms
    err = np.abs(got - y)
    assert (err <= bound + 3 * worst).all(), float(np.max(err - bound - 3 * worst))
    assert np.mean(err <= bound) >= 0.995, float(np.mean(err <= bound))


def test_full_size_int4_decode_layer():
    require_gpu()
    cfg = synth.config_by_name("int4_decode")
    print("[fullsize] int4_decode", flush=True)
    T, E, k, K, N = cfg.T, cfg.E, cfg.topk, cfg.K, cfg.N
    ids, tw = synth.route_inputs(cfg)
    ids_np = ids.numpy()
    tok = 5
    sample, _ = _sample_experts(ids_np, E, tok)
    x = synth.activations(cfg, T, K)
    w = synth.expert_weights(cfg, N, K, device=DEV)
    q4 = torch.empty(E, N, K // 2, dtype=torch.uint8, device=DEV)
    s16 = torch.empty(E, N, K // 128, dtype=torch.float16, device=DEV)
    moe.moe_quant_weight_int4(w, q4, s16)
    kept = {e: u16(w[e]) for e in sample}
    del w
    q4p, s16p = torch.empty_like(q4), torch.empty_like(s16)
    moe.moe_pack_weight_int4(q4, s16, q4p, s16p)
    layer = MoeInt4Layer(q4p, s16p, k, T, moe.LAYOUT_MASKED, cfg.max_m, expected_m=max(1, T * k // E),
                         weights_packed=True)
    z = layer.forward(x.to(DEV), ids.to(DEV), tw.to(DEV))
    torch.cuda.synchronize()
    r = _check_routing(layer, ids_np, E, "masked", cfg.max_m)
    x_bits = u16(x)
    # packing of bf16 rows is a byte copy
    oi = r["output_index"]
    for t in range(T):
        for s in range(k):
            assert np.array_equal(u16(layer.packed[int(oi[t, s])]), x_bits[t])

    cache = {}

    def wfn(e, blocks):
        if e not in cache:
            rows = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
            qq, ss = oracle.quant_weight_int4(kept[e][rows][None])
            rr = torch.from_numpy(rows).to(DEV)
            assert np.array_equal(q4[e][rr].cpu().numpy(), qq[0]), f"int4 codes of expert {e}"
            assert np.array_equal(u16(s16[e][rr]), ss[0]), f"int4 scales of expert {e}"
            cache[e] = oracle.dequant_weight_int4(qq[0], ss[0])
        return cache[e]

    c = dict(T=T, k=k, N=N, K=K, tok=tok, tw=tw.numpy(), sample=sample)
    _fp8_gemm_and_combine(c, r, lambda tt: oracle.bf16_bits_to_f64(x_bits[tt]), layer.D, z, wfn, "int4")


@pytest.mark.parametrize("name", ["dsv3_decode", "dsv3_prefill"])
def test_full_size_int8_variant(name):
    """The benchmark's INT8 (1, 1, 128) variant of a DeepSeek-V3-shaped workload at full size, launched as the
    benchmark launches it (codes and scales routed together, packed weights, tiling hint = routes per expert):
    routing bit-exact on every route, quantisation bit-exact on sampled tokens and weight blocks, packing a byte
    copy, GEMM and combine on sampled outputs."""
    require_gpu()
    cfg = synth.config_by_name(name)
    print(f"[fullsize] int8 {name}", flush=True)
    T, E, k, K, N = cfg.T, cfg.E, cfg.topk, cfg.K, cfg.N
    ids, tw = synth.route_inputs(cfg)
    ids_np = ids.numpy()
    tok = cfg.T // 3 + 2
    sample, _ = _sample_experts(ids_np, E, tok)
    x = synth.activations(cfg, T, K)
    codes = torch.empty(E, N, K, dtype=torch.int8, device=DEV)
    sw = torch.empty(E, K // 128, N, dtype=torch.float32, device=DEV)
    kept = {}
    for e0 in range(0, E, 16):
        ex = list(range(e0, min(E, e0 + 16)))
        w = synth.expert_weights(cfg, N, K, experts=ex, stream=synth.STREAM_WEIGHTS, device=DEV)
        moe.moe_quant_weight_int8(w, codes[e0:e0 + len(ex)], sw[e0:e0 + len(ex)])
        for i, e in enumerate(ex):
            if e in sample:
                kept[e] = u16(w[i])
        del w
    W = torch.empty(E, N, K, dtype=torch.uint8, device=DEV)
    moe.moe_pack_weight_fp8(codes.view(torch.uint8), W)
    layout = moe.LAYOUT_MASKED if cfg.layout == "masked" else moe.LAYOUT_CONTIGUOUS
    am = cfg.max_m if cfg.layout == "masked" else cfg.align
    rows_cap = moe.moe_packed_rows_cap(T, k, E, am) if layout == moe.LAYOUT_CONTIGUOUS else E * am
    em = max(1, T * k // E)
    xd = x.to(DEV)
    q = torch.empty(T, K, dtype=torch.int8, device=DEV)
    sf = torch.empty(T, K // 128, dtype=torch.float32, device=DEV)
    P = torch.empty(rows_cap, K, dtype=torch.int8, device=DEV)
    Psf = torch.empty(rows_cap, K // 128, dtype=torch.float32, device=DEV)
    counts = torch.zeros(E, dtype=torch.int32, device=DEV)
    seg = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    mi = torch.empty(rows_cap, dtype=torch.int32, device=DEV)
    oi = torch.empty(T, k, dtype=torch.int32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(moe.moe_route_pack_workspace_bytes(T, k, E), 16), dtype=torch.uint8, device=DEV)
    D = torch.empty(rows_cap, N, dtype=torch.bfloat16, device=DEV)
    Z = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    moe.moe_quant_act_int8(xd, q, sf)
    moe.moe_route_pack(ids.to(DEV), E, layout, am, q, P, counts, seg, mi, oi, st, payload2=sf, packed2=Psf,
                       workspace=ws)
    am_gemm = am if layout == moe.LAYOUT_MASKED else rows_cap
    moe.moe_grouped_gemm_int8(layout | moe.WEIGHTS_PACKED, P, Psf, W, sw, D, counts, seg, E, am_gemm, N, K, em)
    moe.moe_unpermute_combine(D, oi, tw.to(DEV), Z)
    torch.cuda.synchronize()

    class _L:
        pass

    lay = _L()
    lay.counts, lay.seg_offsets, lay.output_index, lay.m_indices, lay.dev_status = counts, seg, oi, mi, st
    lay.rows_cap = rows_cap
    r = _check_routing(lay, ids_np, E, cfg.layout, am)
    x_bits = u16(x)
    toks = np.array(sorted(set([0, T - 1, tok] + list(range(1, T, max(1, T // 16))))))
    oq, os_ = oracle.quant_int8(x_bits[toks])
    assert np.array_equal(q[torch.from_numpy(toks).to(DEV)].cpu().numpy(), oq)
    assert np.array_equal(sf[torch.from_numpy(toks).to(DEV)].cpu().numpy(), os_)
    oiv = r["output_index"].reshape(-1)
    ok = oiv >= 0
    src = torch.from_numpy((np.arange(oiv.size) // k)[ok].astype(np.int64)).to(DEV)
    dst = torch.from_numpy(oiv[ok].astype(np.int64)).to(DEV)
    assert torch.equal(P[dst], q[src]) and torch.equal(Psf[dst], sf[src])

    cache = {}

    def wfn(e, blocks):
        if e not in cache:
            rows = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
            qq, ss = oracle.quant_int8(kept[e][rows])
            rr = torch.from_numpy(rows).to(DEV)
            assert np.array_equal(codes[e][rr].cpu().numpy(), qq), f"int8 codes of expert {e}"
            assert np.array_equal(sw[e][:, rr].cpu().numpy(), ss.T), f"int8 scales of expert {e}"
            cache[e] = oracle.dequant_int8(qq, ss)
        return cache[e]

    def a_of_tokens(tt):
        a, sa = oracle.quant_int8(x_bits[tt])
        return oracle.dequant_int8(a, sa)

    c = dict(T=T, k=k, N=N, K=K, tok=tok, tw=tw.numpy(), sample=sample)
    _fp8_gemm_and_combine(c, r, a_of_tokens, D, Z, wfn, "fp8")
