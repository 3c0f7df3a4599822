"""GPU routing/packing vs the oracle, bit-exact (all outputs, status bits and payload bytes)."""

import json
import os

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import oracle
import synth
from gpu_helpers import DEV, Routed, oracle_route, require_gpu

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")
SENT = 0xAB


def _check(r: Routed, ids: torch.Tensor, payload: torch.Tensor, payload2=None):
    o = oracle_route(ids, r.E, r.layout, r.am, r.rows_cap)
    torch.cuda.synchronize()
    assert np.array_equal(r.counts.cpu().numpy(), o["counts"])
    assert np.array_equal(r.seg_offsets.cpu().numpy(), o["seg_offsets"])
    assert np.array_equal(r.output_index.cpu().numpy(), o["output_index"])
    assert np.array_equal(r.m_indices.cpu().numpy(), o["m_indices"])
    assert int(r.dev_status.item()) == o["status"]
    # payload rows: every routed row equals its token row; all other rows untouched
    rb = int(np.prod(payload.shape[1:])) * payload.element_size()
    pk = r.packed.view(torch.uint8).reshape(r.rows_cap, rb).cpu().numpy()
    src = payload.view(torch.uint8).reshape(payload.shape[0], rb).cpu().numpy()
    exp = oracle.pack_rows(src, o["output_index"], r.rows_cap, fill=SENT)
    assert np.array_equal(pk, exp)
    if payload2 is not None:
        rb2 = int(np.prod(payload2.shape[1:])) * payload2.element_size()
        pk2 = r.packed2.view(torch.uint8).reshape(r.rows_cap, rb2).cpu().numpy()
        src2 = payload2.view(torch.uint8).reshape(payload2.shape[0], rb2).cpu().numpy()
        assert np.array_equal(pk2, oracle.pack_rows(src2, o["output_index"], r.rows_cap, fill=SENT))
    return o


@pytest.mark.parametrize("align", [1, 128])
def test_worked_example(align):
    require_gpu()
    g = json.load(open(GOLDEN, encoding="utf-8"))
    ids = torch.tensor(g["topk_ids"], dtype=torch.int32, device=DEV)
    x = torch.tensor(g["x"], dtype=torch.float32).to(torch.bfloat16).to(DEV)  # K=8 -> 16-byte rows
    r = Routed(ids, 4, moe.LAYOUT_CONTIGUOUS, align, x, fill=SENT)
    o = _check(r, ids, x)
    key = "unaligned" if align == 1 else "aligned128"
    assert r.output_index.cpu().tolist() == g[key]["output_index"]
    assert int(r.seg_offsets[4].item()) == g[key]["m_packed"]


CASES = [
    # (T, k, E, layout, align/max_m, id range low..high) -- small path (<= 4096 routes) and large path
    (1, 1, 1, 0, 128, 0, 1),
    (37, 3, 9, 0, 16, -2, 11),        # negative and out-of-range ids
    (200, 8, 256, 0, 128, 0, 256),
    (512, 8, 64, 1, 20, 0, 64),       # masked, capacity overflow likely
    (4096, 1, 1024, 0, 128, 0, 1024),
    (1000, 8, 64, 0, 128, -1, 66),    # large path with invalid ids
    (3000, 8, 96, 1, 300, 0, 96),     # large path, masked with overflow
    (0, 4, 8, 0, 128, 0, 8),          # empty
]


@pytest.mark.parametrize("case", CASES)
def test_random_routing_bit_exact(case):
    require_gpu()
    T, k, E, layout, am, lo, hi = case
    g = torch.Generator().manual_seed(T * 131 + k * 7 + E)
    ids = torch.randint(lo, hi, (T, k), generator=g, dtype=torch.int32)
    K = 256
    codes = torch.randint(0, 256, (T, K), generator=g, dtype=torch.int32).to(torch.uint8)
    scales = torch.rand(T, K // 128, generator=g, dtype=torch.float32)
    r = Routed(ids.to(DEV), E, layout, am, codes.to(DEV), payload2=scales.to(DEV), fill=SENT)
    _check(r, ids, codes, scales)


def test_full_size_routing(tmp_path):
    """Routing and packing at the DeepSeek-V3 and Qwen3 prefill sizes (FP8 rows + scale rows)."""
    require_gpu()
    for name in ("dsv3_prefill", "qwen3_skewed", "dsv3_decode", "int4_decode"):
        cfg = synth.config_by_name(name)
        ids, _ = synth.route_inputs(cfg)
        layout = moe.LAYOUT_MASKED if cfg.layout == "masked" else moe.LAYOUT_CONTIGUOUS
        am = cfg.max_m if cfg.layout == "masked" else cfg.align
        gen = torch.Generator(device=DEV).manual_seed(1)
        if cfg.weights == "int4":
            payload = torch.randn(cfg.T, cfg.K, device=DEV, generator=gen).to(torch.bfloat16)
            payload2 = None
        else:
            payload = torch.randint(0, 256, (cfg.T, cfg.K), device=DEV, generator=gen, dtype=torch.int32).to(torch.uint8)
            payload2 = torch.rand(cfg.T, cfg.K // 128, device=DEV, generator=gen)
        r = Routed(ids.to(DEV), cfg.E, layout, am, payload, payload2=payload2, fill=SENT)
        _check(r, ids, payload, payload2)


def test_determinism_20_runs():
    require_gpu()
    g = torch.Generator().manual_seed(9)
    ids = torch.randint(0, 64, (2000, 8), generator=g, dtype=torch.int32).to(DEV)
    payload = torch.randint(0, 256, (2000, 128), generator=g, dtype=torch.int32).to(torch.uint8).to(DEV)
    ref = Routed(ids, 64, moe.LAYOUT_CONTIGUOUS, 128, payload, fill=0)
    for _ in range(20):
        r = Routed(ids, 64, moe.LAYOUT_CONTIGUOUS, 128, payload, fill=0)
        for a, b in ((r.output_index, ref.output_index), (r.packed, ref.packed), (r.m_indices, ref.m_indices),
                     (r.seg_offsets, ref.seg_offsets)):
            assert torch.equal(a, b)


def test_quant_then_gather_equals_gather_then_quant():
    """Quantisation is row-local, so packing quantised rows equals quantising packed rows."""
    require_gpu()
    from gpu_helpers import fp8_quant_gpu
    g = torch.Generator().manual_seed(10)
    x = torch.randn(300, 512, generator=g).to(torch.bfloat16).to(DEV)
    ids = torch.randint(0, 16, (300, 4), generator=g, dtype=torch.int32).to(DEV)
    q, sf = fp8_quant_gpu(x)
    r1 = Routed(ids, 16, moe.LAYOUT_CONTIGUOUS, 128, q, payload2=sf, fill=0)
    r2 = Routed(ids, 16, moe.LAYOUT_CONTIGUOUS, 128, x, fill=0)
    q2, sf2 = fp8_quant_gpu(r2.packed)
    rows = torch.nonzero(r1.m_indices >= 0).flatten()
    oi = r1.output_index.flatten()
    used = oi[oi >= 0].long()
    assert torch.equal(r1.packed[used], q2[used]) and torch.equal(r1.packed2[used], sf2[used])
    assert rows.numel() >= used.numel()


def _route_quant(ids, E, layout, am, x, fill=SENT):
    """One moe_route_pack_quant call (sentinel-filled outputs)."""
    T, k = ids.shape
    K = x.shape[1]
    rows_cap = moe.moe_packed_rows_cap(T, k, E, am) if layout == moe.LAYOUT_CONTIGUOUS else E * am
    r = type("RQ", (), {})()
    r.E, r.layout, r.am, r.rows_cap = E, layout, am, rows_cap
    r.packed = torch.full((rows_cap, K), fill, dtype=torch.uint8, device=DEV)
    r.packed2 = torch.empty(rows_cap, K // 128, dtype=torch.float32, device=DEV)
    r.packed2.view(torch.uint8).fill_(fill)
    r.counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    r.seg_offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    r.m_indices = torch.full((rows_cap,), -7, dtype=torch.int32, device=DEV)
    r.output_index = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    r.dev_status = torch.zeros(1, dtype=torch.int32, device=DEV)
    wsb = moe.moe_route_pack_workspace_bytes(T, k, E)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=DEV) if wsb > 0 else None
    moe.moe_route_pack_quant(ids, E, layout, am, x, r.packed, r.packed2, r.counts, r.seg_offsets, r.m_indices,
                             r.output_index, r.dev_status, workspace=ws)
    torch.cuda.synchronize()
    return r


QUANT_CASES = [
    # (T, k, E, layout, align/max_m, id low..high, K): single-launch and multi-launch paths
    (1, 1, 1, 0, 128, 0, 1, 128),
    (37, 3, 9, 0, 16, -2, 11, 384),      # negative and out-of-range ids
    (512, 8, 64, 1, 20, 0, 64, 256),     # masked, capacity overflow
    (600, 8, 64, 0, 128, -1, 66, 4352),  # multi-launch path (4800 routes), 34 blocks per row (a partial group of 32)
    (700, 8, 96, 1, 40, 0, 96, 1024),    # multi-launch, masked with overflow
    (0, 4, 8, 0, 128, 0, 8, 256),        # empty
    (60, 64, 1024, 0, 128, 0, 1024, 128),  # the largest k and E, one block per row
    (5, 2, 3, 1, 8, 0, 3, 32768),        # the largest K (256 blocks per row: every scale slot of the kernel)
]


@pytest.mark.parametrize("case", QUANT_CASES)
def test_route_pack_quant_equals_quant_then_pack(case):
    """The quantising pack against the oracle (routing outputs and, for every route, the oracle's 1x128 codes and
    scales of its token row; untouched padding rows) and against moe_quant_act followed by moe_route_pack, bit for
    bit."""
    require_gpu()
    from gpu_helpers import fp8_quant_gpu
    T, k, E, layout, am, lo, hi, K = case
    g = torch.Generator().manual_seed(T * 17 + k + E + K)
    ids = torch.randint(lo, hi, (T, k), generator=g, dtype=torch.int32)
    x = (torch.randn(T, K, generator=g) * torch.exp2(torch.randint(-8, 9, (T, 1), generator=g).float()))
    x = x.to(torch.bfloat16)
    if T > 2:
        x[1, :128] = 0.0                      # an all-zero block
        x[2, 128 % K:] *= 1e-30               # tiny values
    r = _route_quant(ids.to(DEV), E, layout, am, x.to(DEV))
    o = oracle_route(ids, E, layout, am, r.rows_cap)
    assert np.array_equal(r.counts.cpu().numpy(), o["counts"])
    assert np.array_equal(r.seg_offsets.cpu().numpy(), o["seg_offsets"])
    assert np.array_equal(r.output_index.cpu().numpy(), o["output_index"])
    assert np.array_equal(r.m_indices.cpu().numpy(), o["m_indices"])
    assert int(r.dev_status.item()) == o["status"]
    xb = x.view(torch.int16).numpy().view(np.uint16)
    q_o, s_o = oracle.quant_act(xb) if T > 0 else (np.zeros((0, K), np.uint8), np.zeros((0, K // 128), np.float32))
    assert np.array_equal(r.packed.cpu().numpy(), oracle.pack_rows(q_o, o["output_index"], r.rows_cap, fill=SENT))
    sf_bytes = s_o.view(np.uint8).reshape(T, 4 * (K // 128))
    got_sf = r.packed2.view(torch.uint8).cpu().numpy()
    assert np.array_equal(got_sf, oracle.pack_rows(sf_bytes, o["output_index"], r.rows_cap, fill=SENT))
    if T > 0:
        q, sf = fp8_quant_gpu(x.to(DEV))
        chain = Routed(ids.to(DEV), E, layout, am, q, payload2=sf, fill=SENT)
        assert torch.equal(chain.packed, r.packed) and torch.equal(chain.packed2.view(torch.uint8),
                                                                   r.packed2.view(torch.uint8))
        assert torch.equal(chain.output_index, r.output_index) and torch.equal(chain.m_indices, r.m_indices)
