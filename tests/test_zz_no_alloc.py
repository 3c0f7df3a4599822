"""moe_route_pack_noalloc (the fixed device scratch) against moe_route_pack (a caller's workspace).

Two calls in a row on one device, the second with a smaller input, both on
the multi-launch path that uses the scratch (T*k > 4096 routes), then one on
the single-launch path; every output must equal moe_route_pack's bit for bit.
"""

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import synth
from gpu_helpers import DEV, Routed, require_gpu

pytestmark = pytest.mark.gpu


def _noalloc(ids, E, layout, am, payload, payload2, rows_cap, fill):
    T, k = ids.shape
    packed = torch.empty((rows_cap,) + tuple(payload.shape[1:]), dtype=payload.dtype, device=DEV)
    packed.view(torch.uint8).fill_(fill)
    packed2 = torch.empty((rows_cap,) + tuple(payload2.shape[1:]), dtype=payload2.dtype, device=DEV)
    packed2.view(torch.uint8).fill_(fill)
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    seg = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    mi = torch.full((rows_cap,), -7, dtype=torch.int32, device=DEV)
    oi = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    moe.moe_route_pack_noalloc(ids, E, layout, am, payload, packed, counts, seg, mi, oi, st, payload2=payload2,
                               packed2=packed2)
    return dict(packed=packed, packed2=packed2, counts=counts, seg_offsets=seg, m_indices=mi, output_index=oi,
                dev_status=st)


def _case(name, T, E, layout, am, seed):
    cfg = synth.config_by_name(name)
    ids, _ = synth.route_inputs(cfg, seed=seed, T=T)
    ids = ids.clone()
    if E < cfg.E:
        ids = ids % E
    ids[0, 0] = E + 3          # an id out of range: skipped and flagged
    ids[1, 1] = -1             # a negative id: skipped
    payload = torch.randint(0, 256, (T, 256), dtype=torch.uint8, device=DEV)
    payload2 = torch.randn(T, 2, device=DEV)
    return ids.to(DEV), payload, payload2


def _compare(ids, E, layout, am, payload, payload2):
    ref = Routed(ids, E, layout, am, payload, payload2=payload2, fill=0x5A)
    got = _noalloc(ids, E, layout, am, payload, payload2, ref.rows_cap, 0x5A)
    torch.cuda.synchronize()
    for key in ("counts", "seg_offsets", "m_indices", "output_index", "dev_status", "packed", "packed2"):
        a, b = getattr(ref, key), got[key]
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                           b.view(torch.uint8) if b.dtype != torch.int32 else b), key
    return ref


def test_noalloc_matches_workspace_call_twice_then_smaller():
    require_gpu()
    assert moe.moe_route_pack_noalloc_max_bytes() == 4 << 20
    print("[no_alloc] qwen3-shaped routing, T=8192 E=128 contiguous", flush=True)
    ids, p, p2 = _case("qwen3_skewed", 8192, 128, moe.LAYOUT_CONTIGUOUS, 128, 0)
    r = _compare(ids, 128, moe.LAYOUT_CONTIGUOUS, 128, p, p2)
    assert int(r.dev_status.item()) == moe.DEV_ID_RANGE
    print("[no_alloc] second call, smaller: T=1024 E=64 masked max_m=256", flush=True)
    ids, p, p2 = _case("dsv3_prefill", 1024, 64, moe.LAYOUT_MASKED, 256, 1)
    _compare(ids, 64, moe.LAYOUT_MASKED, 256, p, p2)
    print("[no_alloc] third call, single-launch path: T=100 E=16", flush=True)
    ids, p, p2 = _case("dsv3_prefill", 100, 16, moe.LAYOUT_CONTIGUOUS, 128, 2)
    _compare(ids, 16, moe.LAYOUT_CONTIGUOUS, 128, p, p2)


def test_noalloc_refuses_more_than_its_scratch():
    require_gpu()
    # 2^20 tokens x 8 routes over 1024 experts would need ~33 MB of scratch: refused before any launch
    T, k, E = 1 << 20, 8, 1024
    need = moe.moe_route_pack_workspace_bytes(T, k, E)
    assert need > moe.moe_route_pack_noalloc_max_bytes()
    ids = torch.zeros(1, dtype=torch.int32, device=DEV)
    lib = moe.load()
    import ctypes
    p = ctypes.c_void_p(ids.data_ptr())
    rows_cap = moe.moe_packed_rows_cap(T, k, E, 128)
    st = lib.moe_route_pack_noalloc(p, T, k, E, 0, 128, p, 16, None, 0, p, None, rows_cap, p, p, p, p, p, None)
    assert st == 6 and b"scratch" in lib.moe_last_error()
