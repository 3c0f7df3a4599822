"""The C ABI: libmoe.so loads, exports every entry point include/moe.h declares,
and rejects bad arguments on the host before launching anything (CPU only)."""

import ctypes
import os
import re

import pytest

import int4_weights_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGN, MOE_ERR_HIP, MOE_ERR_WORKSPACE = range(7)


def _declared():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return moe.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert set(names) == set(moe.SIGNATURES)


def test_constants_and_helpers(lib):
    assert moe.moe_abi_version() == 2
    assert lib.moe_status_str(MOE_ERR_WORKSPACE) == b"workspace missing or too small"
    # worked example: 10 routes, 4 experts, 128-aligned -> at most 640 rows
    assert moe.moe_packed_rows_cap(5, 2, 4, 128) == 640
    assert moe.moe_packed_rows_cap(4096, 8, 256, 128) == 65280
    assert moe.moe_packed_rows_cap(0, 8, 256, 128) == 0
    assert moe.moe_packed_rows_cap(1, 0, 4, 128) == -1
    assert moe.moe_route_pack_workspace_bytes(128, 8, 256) == 0
    assert moe.moe_route_pack_workspace_bytes(4096, 8, 256) == 4 * (32 * 256 + 32)
    assert moe.moe_route_pack_workspace_bytes(1, 1, 2000) == -1


def _p(v):
    return ctypes.c_void_p(v)


def moe_cap(lib, T, k, E, align):
    return lib.moe_packed_rows_cap(T, k, E, align)


A16 = 1 << 20  # a fake, 16-byte aligned address: never dereferenced on these error paths


def test_host_validation_rejects_without_launching(lib):
    # moe_quant_act
    assert lib.moe_quant_act(_p(A16), 4, 100, _p(A16), _p(A16), None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_quant_act(None, 4, 128, _p(A16), _p(A16), None) == MOE_ERR_NULL
    assert lib.moe_quant_act(_p(A16 + 2), 4, 128, _p(A16), _p(A16), None) == MOE_ERR_ALIGN
    assert lib.moe_quant_act(_p(A16), -1, 128, _p(A16), _p(A16), None) == MOE_ERR_SHAPE
    assert lib.moe_quant_act(None, 0, 128, None, None, None) == MOE_OK  # empty input is a no-op
    assert b"multiple of 128" in (lib.moe_quant_act(_p(A16), 4, 100, _p(A16), _p(A16), None) and
                                  lib.moe_last_error())
    # moe_quant_weight_*
    assert lib.moe_quant_weight_fp8(_p(A16), 2, 100, 128, _p(A16), _p(A16), None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_quant_weight_int4(_p(A16), 2, 128, 64, _p(A16), _p(A16), None) == MOE_ERR_UNSUPPORTED
    # moe_pack_weight_fp8: shape, alignment, overlap
    assert lib.moe_pack_weight_fp8(_p(A16), 2, 100, 128, _p(A16 << 4), None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_pack_weight_fp8(_p(A16 + 8), 2, 128, 128, _p(A16 << 4), None) == MOE_ERR_ALIGN
    assert lib.moe_pack_weight_fp8(None, 2, 128, 128, _p(A16 << 4), None) == MOE_ERR_NULL
    assert lib.moe_pack_weight_fp8(_p(A16), 2, 128, 128, _p(A16 + 4096), None) == MOE_ERR_SHAPE  # overlap
    assert lib.moe_pack_weight_fp8(None, 0, 128, 128, None, None) == MOE_OK  # no experts: no-op

    # moe_route_pack
    def rp(T=5, k=2, E=4, layout=0, am=128, rb=16, rows_cap=640, ws=None, wsb=0, payload=A16, ids=A16):
        return lib.moe_route_pack(_p(ids) if ids else None, T, k, E, layout, am, _p(payload) if payload else None,
                                  rb, None, 0, _p(A16), None, rows_cap, _p(A16), _p(A16), _p(A16), _p(A16),
                                  _p(A16), _p(ws) if ws else None, wsb, None)

    assert rp(E=0) == MOE_ERR_SHAPE
    assert rp(E=1025) == MOE_ERR_SHAPE
    assert rp(k=0) == MOE_ERR_SHAPE
    assert rp(layout=7) == MOE_ERR_SHAPE
    assert rp(am=0) == MOE_ERR_SHAPE
    assert rp(rb=6) == MOE_ERR_ALIGN
    assert rp(payload=0) == MOE_ERR_NULL
    assert rp(rows_cap=639) == MOE_ERR_SHAPE          # below the packed-rows bound
    assert rp(layout=1, am=3, rows_cap=11) == MOE_ERR_SHAPE  # masked needs E*max_m rows
    assert rp(payload=A16 + 4) == MOE_ERR_ALIGN
    assert rp(T=4096, k=8, E=256, rows_cap=65280) == MOE_ERR_WORKSPACE  # large path needs scratch
    assert rp(T=4096, k=8, E=256, rows_cap=65280, ws=A16, wsb=100) == MOE_ERR_WORKSPACE

    # moe_grouped_gemm_fp8 / int4
    def g8(layout=0, N=256, K=256, E=4, rows=512, seg=A16, A=A16):
        return lib.moe_grouped_gemm_fp8(layout, _p(A) if A else None, _p(A16), _p(A16), _p(A16), _p(A16), _p(A16),
                                        _p(seg) if seg else None, E, rows, N, K, 0, None)

    assert g8(N=200) == MOE_ERR_UNSUPPORTED
    assert g8(K=100) == MOE_ERR_UNSUPPORTED
    assert g8(E=0) == MOE_ERR_SHAPE
    assert g8(seg=0) == MOE_ERR_NULL                 # contiguous needs seg_offsets
    assert g8(A=0) == MOE_ERR_NULL
    assert g8(A=A16 + 8) == MOE_ERR_ALIGN
    assert g8(K=128 * 300) == MOE_ERR_UNSUPPORTED    # K above the supported maximum
    assert g8(layout=0x10 | 7) == MOE_ERR_SHAPE      # the packed-weights flag does not make a layout valid
    assert g8(layout=0x10, seg=0) == MOE_ERR_NULL    # packed contiguous still needs seg_offsets
    assert lib.moe_grouped_gemm_int4(0x10 | 7, _p(A16), _p(A16), _p(A16), _p(A16), _p(A16), _p(A16), 4, 64, 128,
                                     256, 0, None) == MOE_ERR_SHAPE  # the flag does not make a layout valid
    # moe_pack_weight_int4(q4, s16, E, N, K, q4_packed, s16_packed, stream)
    def p4(q=A16, sc=A16 << 2, E=2, N=128, K=128, qo=A16 << 4, so=A16 << 6):
        return lib.moe_pack_weight_int4(_p(q) if q else None, _p(sc) if sc else None, E, N, K, _p(qo) if qo else None,
                                        _p(so) if so else None, None)

    assert p4(N=100) == MOE_ERR_UNSUPPORTED
    assert p4(K=64) == MOE_ERR_UNSUPPORTED
    assert p4(q=A16 + 8) == MOE_ERR_ALIGN
    assert p4(so=(A16 << 6) + 2) == MOE_ERR_ALIGN
    assert p4(q=0) == MOE_ERR_NULL
    assert p4(so=0) == MOE_ERR_NULL
    assert p4(qo=A16 + 4096) == MOE_ERR_SHAPE         # weights in and out overlap
    assert p4(so=A16 + 4096) == MOE_ERR_SHAPE         # scales out overlap weights in
    assert p4(so=(A16 << 4) + 256) == MOE_ERR_SHAPE   # the two outputs overlap
    assert p4(q=0, sc=0, E=0, qo=0, so=0) == MOE_OK
    assert lib.moe_grouped_gemm_int4(0, _p(A16), _p(A16), _p(A16), _p(A16), _p(A16), _p(A16), 4, 64, 100, 256, 0,
                                     None) == MOE_ERR_UNSUPPORTED
    # packed 4-bit scales are read 8 bytes at a time: a 4-byte aligned S16 is refused with packed weights only
    # (a valid call would launch, so the accepted case is checked as not refused for alignment on the GPU)
    assert lib.moe_grouped_gemm_int4(0x10 | 1, _p(A16), _p(A16), _p(A16 + 4), _p(A16), _p(A16), _p(A16), 4, 64, 128,
                                     256, 0, None) == MOE_ERR_ALIGN
    assert lib.moe_grouped_gemm_int4(1, _p(A16), _p(A16), _p(A16 + 3), _p(A16), _p(A16), _p(A16), 4, 64, 128,
                                     256, 0, None) == MOE_ERR_ALIGN
    # moe_route_pack_noalloc: the same checks as moe_route_pack, and a refusal (before any launch) of calls
    # whose scratch would exceed the fixed 4 MiB array
    assert lib.moe_route_pack_noalloc_max_bytes() == 4 << 20

    def rpn(T=5, k=2, E=4, layout=0, am=128, rb=16, rows_cap=640, payload=A16):
        return lib.moe_route_pack_noalloc(_p(A16), T, k, E, layout, am, _p(payload) if payload else None, rb, None, 0,
                                          _p(A16), None, rows_cap, _p(A16), _p(A16), _p(A16), _p(A16), _p(A16), None)

    assert rpn(layout=7) == MOE_ERR_SHAPE
    assert rpn(rb=6) == MOE_ERR_ALIGN
    assert rpn(payload=0) == MOE_ERR_NULL
    assert rpn(rows_cap=100) == MOE_ERR_SHAPE
    big_T = 1 << 20
    assert rpn(T=big_T, k=8, E=1024, rows_cap=lib.moe_packed_rows_cap(big_T, 8, 1024, 128)) == MOE_ERR_WORKSPACE
    assert b"scratch" in lib.moe_last_error()
    # moe_grouped_gemm_bf16(layout, A, W, D, counts, seg, E, rows, N, K, expected_m, stream)
    def gb(layout=0, N=256, K=256, E=4, rows=512, seg=A16, A=A16, W=A16):
        return lib.moe_grouped_gemm_bf16(layout, _p(A) if A else None, _p(W) if W else None, _p(A16), _p(A16),
                                         _p(seg) if seg else None, E, rows, N, K, 0, None)

    assert gb(N=200) == MOE_ERR_UNSUPPORTED
    assert gb(K=64) == MOE_ERR_UNSUPPORTED
    assert gb(E=0) == MOE_ERR_SHAPE
    assert gb(layout=0x10 | 7) == MOE_ERR_SHAPE      # the packed-weights flag does not make a layout valid
    assert lib.moe_pack_weight_bf16(_p(A16), 2, 100, 128, _p(A16 << 4), None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_pack_weight_bf16(_p(A16 + 8), 2, 128, 128, _p(A16 << 4), None) == MOE_ERR_ALIGN
    assert lib.moe_pack_weight_bf16(_p(A16), 2, 128, 128, _p(A16 + 4096), None) == MOE_ERR_SHAPE  # overlap
    assert lib.moe_pack_weight_bf16(None, 0, 128, 128, None, None) == MOE_OK
    assert gb(seg=0) == MOE_ERR_NULL
    assert gb(W=0) == MOE_ERR_NULL
    assert gb(A=A16 + 8) == MOE_ERR_ALIGN
    assert gb(K=128 * 300) == MOE_ERR_UNSUPPORTED
    # moe_stream_read(buf, bytes, out, stream): the measurement helper validates like the path's calls
    assert lib.moe_stream_read(_p(A16), 100, _p(A16), None) == MOE_ERR_SHAPE
    assert lib.moe_stream_read(_p(A16), -16, _p(A16), None) == MOE_ERR_SHAPE
    assert lib.moe_stream_read(_p(A16), 64, None, None) == MOE_ERR_NULL
    assert lib.moe_stream_read(None, 64, _p(A16), None) == MOE_ERR_NULL
    assert lib.moe_stream_read(_p(A16 + 8), 64, _p(A16), None) == MOE_ERR_ALIGN
    assert lib.moe_stream_read(_p(A16), 64, _p(A16 + 2), None) == MOE_ERR_ALIGN
    # moe_grouped_gemm_fp8_fp4(layout, A, SFA, W4, SW, D, counts, seg, E, rows, N, K, expected_m, stream)
    def g4(layout=0, N=256, K=256, E=4, rows=512, seg=A16, A=A16, SW=A16, SFA=A16):
        return lib.moe_grouped_gemm_fp8_fp4(layout, _p(A) if A else None, _p(SFA) if SFA else None, _p(A16),
                                            _p(SW) if SW else None, _p(A16), _p(A16), _p(seg) if seg else None, E,
                                            rows, N, K, 0, None)

    assert g4(N=200) == MOE_ERR_UNSUPPORTED
    assert g4(K=192) == MOE_ERR_UNSUPPORTED
    assert g4(layout=0x10 | 7) == MOE_ERR_SHAPE         # the packed-weights flag does not make a layout valid
    assert g4(seg=0) == MOE_ERR_NULL
    assert g4(SFA=0) == MOE_ERR_NULL
    assert g4(SW=0) == MOE_ERR_NULL
    assert g4(SW=A16 + 2) == MOE_ERR_ALIGN
    assert g4(A=A16 + 8) == MOE_ERR_ALIGN
    def pf4(q=A16, sc=A16 << 2, E=2, N=128, K=512, qo=A16 << 4, so=A16 << 6):
        return lib.moe_pack_weight_fp4(_p(q) if q else None, _p(sc) if sc else None, E, N, K, _p(qo) if qo else None,
                                       _p(so) if so else None, None)

    assert pf4(K=320) == MOE_ERR_UNSUPPORTED
    assert pf4(N=100) == MOE_ERR_UNSUPPORTED
    assert pf4(qo=A16 + 8) == MOE_ERR_ALIGN
    assert pf4(so=(A16 << 6) + 2) == MOE_ERR_ALIGN
    assert pf4(sc=0) == MOE_ERR_NULL
    assert pf4(qo=A16 + 4096) == MOE_ERR_SHAPE        # codes out overlap codes in
    assert pf4(q=0, sc=0, E=0, qo=0, so=0) == MOE_OK
    assert lib.moe_quant_weight_fp4(_p(A16), 2, 128, 100, _p(A16), _p(A16), None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_quant_weight_fp4(_p(A16 + 8), 2, 128, 128, _p(A16), _p(A16), None) == MOE_ERR_ALIGN
    assert lib.moe_quant_weight_fp4(None, 2, 128, 128, _p(A16), _p(A16), None) == MOE_ERR_NULL
    assert lib.moe_quant_weight_fp4(None, 0, 128, 128, None, None, None) == MOE_OK
    # moe_swiglu_quant(layout, gate_up, rows_or_max_m, I, counts, seg_offsets, E, q, sf, stream)
    def sw(layout=0, gu=A16, rows=512, I=256, seg=A16, E=4, q=A16, sf=A16):
        return lib.moe_swiglu_quant(layout, _p(gu) if gu else None, rows, I, _p(A16), _p(seg) if seg else None, E,
                                    _p(q) if q else None, _p(sf) if sf else None, None)

    assert sw(I=200) == MOE_ERR_UNSUPPORTED
    assert sw(layout=3) == MOE_ERR_SHAPE
    assert sw(E=0) == MOE_ERR_SHAPE
    assert sw(rows=0) == MOE_ERR_SHAPE
    assert sw(gu=0) == MOE_ERR_NULL
    assert sw(seg=0) == MOE_ERR_NULL                 # contiguous needs seg_offsets
    assert sw(q=A16 + 8) == MOE_ERR_ALIGN
    assert sw(sf=A16 + 2) == MOE_ERR_ALIGN
    # moe_grouped_gemm_fp8_swiglu(layout, A, SFA, W, SFW, Q, SQ, counts, seg, E, rows, I, K, expected_m, stream)
    def gs(layout=0, I=256, K=512, E=4, rows=512, seg=A16, A=A16, SFA=A16, SQ=A16, Q=A16):
        return lib.moe_grouped_gemm_fp8_swiglu(layout, _p(A) if A else None, _p(SFA) if SFA else None, _p(A16),
                                               _p(A16), _p(Q) if Q else None, _p(SQ) if SQ else None, _p(A16),
                                               _p(seg) if seg else None, E, rows, I, K, 0, None)

    assert gs(I=192) == MOE_ERR_UNSUPPORTED          # I must be a multiple of 128 (N = 2I of 256)
    assert gs(I=0) == MOE_ERR_SHAPE
    assert gs(K=384) == MOE_ERR_UNSUPPORTED          # the tall tile needs K % 512 == 0
    assert gs(K=100) == MOE_ERR_UNSUPPORTED
    assert gs(layout=0x10 | 7) == MOE_ERR_SHAPE
    assert gs(E=0) == MOE_ERR_SHAPE
    assert gs(seg=0) == MOE_ERR_NULL
    assert gs(SFA=0) == MOE_ERR_NULL
    assert gs(SQ=0) == MOE_ERR_NULL
    assert gs(Q=0) == MOE_ERR_NULL
    assert gs(Q=A16 + 8) == MOE_ERR_ALIGN
    assert gs(SFA=A16 + 4) == MOE_ERR_ALIGN          # row scales: 16-byte copies
    assert gs(SQ=A16 + 2) == MOE_ERR_ALIGN
    # moe_route_pack_quant(ids, T, k, E, layout, am, x, K, packed_q, packed_sf, rows_cap, counts, seg, mi, oi,
    #                      status, ws, ws_bytes, stream)
    def rq(T=5, k=2, E=4, layout=0, am=128, K=256, x=A16, pq=A16 << 4, psf=A16 << 6, rows_cap=640, ids=A16):
        return lib.moe_route_pack_quant(_p(ids) if ids else None, T, k, E, layout, am, _p(x) if x else None, K,
                                        _p(pq) if pq else None, _p(psf) if psf else None, rows_cap, _p(A16),
                                        _p(A16), _p(A16), _p(A16), _p(A16), None, 0, None)

    assert rq(K=200) == MOE_ERR_UNSUPPORTED
    assert rq(K=0) == MOE_ERR_UNSUPPORTED
    assert rq(K=257 * 128) == MOE_ERR_UNSUPPORTED       # more 128-blocks than a row's scales the kernel stages
    assert rq(x=0) == MOE_ERR_NULL
    assert rq(psf=0) == MOE_ERR_NULL
    assert rq(pq=0) == MOE_ERR_NULL
    assert rq(x=A16 + 8) == MOE_ERR_ALIGN
    assert rq(pq=(A16 << 4) + 8) == MOE_ERR_ALIGN
    assert rq(psf=(A16 << 6) + 2) == MOE_ERR_ALIGN
    assert rq(rows_cap=100) == MOE_ERR_SHAPE           # below what the routes need
    assert rq(layout=3) == MOE_ERR_SHAPE
    assert rq(T=5000, k=8, rows_cap=moe_cap(lib, 5000, 8, 4, 128)) == MOE_ERR_WORKSPACE  # multi-launch path, no workspace
    # moe_quant_act_int8 / moe_quant_weight_int8
    assert lib.moe_quant_act_int8(_p(A16), 4, 100, _p(A16), _p(A16), None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_quant_act_int8(None, 4, 128, _p(A16), _p(A16), None) == MOE_ERR_NULL
    assert lib.moe_quant_act_int8(_p(A16), 4, 128, _p(A16 + 8), _p(A16), None) == MOE_ERR_ALIGN
    assert lib.moe_quant_act_int8(_p(A16), 4, 128, _p(A16), _p(A16 + 2), None) == MOE_ERR_ALIGN
    assert lib.moe_quant_act_int8(_p(A16), -1, 128, _p(A16), _p(A16), None) == MOE_ERR_SHAPE
    assert lib.moe_quant_act_int8(None, 0, 128, None, None, None) == MOE_OK
    assert lib.moe_quant_weight_int8(_p(A16), 2, 100, 128, _p(A16), _p(A16), None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_quant_weight_int8(_p(A16), 2, 128, 192, _p(A16), _p(A16), None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_quant_weight_int8(_p(A16 + 2), 2, 128, 128, _p(A16), _p(A16), None) == MOE_ERR_ALIGN
    assert lib.moe_quant_weight_int8(None, 2, 128, 128, _p(A16), _p(A16), None) == MOE_ERR_NULL
    assert lib.moe_quant_weight_int8(None, 0, 128, 128, None, None, None) == MOE_OK
    # moe_grouped_gemm_int8(layout, A, SA, W, SW, D, counts, seg, E, rows, N, K, expected_m, stream)
    def g8(layout=0, N=256, K=256, E=4, rows=512, seg=A16, A=A16, SA=A16, SW=A16, D=A16):
        return lib.moe_grouped_gemm_int8(layout, _p(A) if A else None, _p(SA) if SA else None, _p(A16),
                                         _p(SW) if SW else None, _p(D) if D else None, _p(A16),
                                         _p(seg) if seg else None, E, rows, N, K, 0, None)

    assert g8(N=200) == MOE_ERR_UNSUPPORTED
    assert g8(K=192) == MOE_ERR_UNSUPPORTED
    assert g8(layout=0x10 | 7) == MOE_ERR_SHAPE
    assert g8(E=0) == MOE_ERR_SHAPE
    assert g8(rows=0) == MOE_ERR_SHAPE
    assert g8(seg=0) == MOE_ERR_NULL
    assert g8(SA=0) == MOE_ERR_NULL
    assert g8(SW=0) == MOE_ERR_NULL
    assert g8(D=0) == MOE_ERR_NULL
    assert g8(A=A16 + 8) == MOE_ERR_ALIGN
    assert g8(SA=A16 + 2) == MOE_ERR_ALIGN
    assert g8(SW=A16 + 4) == MOE_ERR_ALIGN            # 4 columns' scales per 16-byte load
    # moe_unpermute_combine
    assert lib.moe_unpermute_combine(_p(A16), 10, _p(A16), _p(A16), 4, 2, 12, _p(A16), None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_unpermute_combine(_p(A16), 10, _p(A16), _p(A16), 4, 0, 16, _p(A16), None) == MOE_ERR_SHAPE
    assert lib.moe_unpermute_combine(_p(A16), 10, None, _p(A16), 4, 2, 16, _p(A16), None) == MOE_ERR_NULL
    assert lib.moe_unpermute_combine(None, 0, None, None, 0, 2, 16, None, None) == MOE_OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.moe_quant_act(x, torch.zeros(4, 128, dtype=torch.uint8), torch.zeros(4, 1))


def test_missing_library_fails_loudly(tmp_path):
    from int4_weights_amd import _lib
    with pytest.raises(ImportError):
        _lib.load.__wrapped__ if hasattr(_lib.load, "__wrapped__") else None
        saved = _lib._lib
        _lib._lib = None
        try:
            _lib.load(str(tmp_path / "nope.so"))
        finally:
            _lib._lib = saved
