"""ctypes binding of libmoe.so: argument marshalling only.

Every function has the name of the C entry point it calls (include/moe.h),
takes torch tensors that already live on the GPU, passes their data pointers
and the current HIP stream, and raises MoeError on a nonzero status.  No
computation happens here; there is no fallback if the library is missing.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

LAYOUT_CONTIGUOUS = 0
LAYOUT_MASKED = 1
WEIGHTS_PACKED = 0x10  # flag for moe_grouped_gemm_fp8's layout: W in moe_pack_weight_fp8 order
DEV_ID_RANGE = 1
DEV_CAPACITY = 2

_c_i32, _c_i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p

# name -> (restype, argtypes)
SIGNATURES = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_status_str": (ctypes.c_char_p, [_c_i32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_packed_rows_cap": (_c_i64, [ctypes.c_int] * 4),
    "moe_route_pack_workspace_bytes": (_c_i64, [ctypes.c_int] * 3),
    "moe_quant_act": (_c_i32, [_vp, _c_i64, ctypes.c_int, _vp, _vp, _vp]),
    "moe_quant_weight_fp8": (_c_i32, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]),
    "moe_quant_weight_int4": (_c_i32, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]),
    "moe_pack_weight_fp8": (_c_i32, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp]),
    "moe_pack_weight_int4": (_c_i32, [_vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]),
    "moe_route_pack": (_c_i32, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                _vp, _c_i64, _vp, _c_i64, _vp, _vp, _c_i64,
                                _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "moe_route_pack_quant": (_c_i32, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      _vp, ctypes.c_int, _vp, _vp, _c_i64,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "moe_route_pack_noalloc_max_bytes": (_c_i64, []),
    "moe_route_pack_noalloc": (_c_i32, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        _vp, _c_i64, _vp, _c_i64, _vp, _vp, _c_i64,
                                        _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_grouped_gemm_fp8": (_c_i32, [ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_int, _c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]),
    "moe_grouped_gemm_fp8_swiglu": (_c_i32, [ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             ctypes.c_int, _c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]),
    "moe_grouped_gemm_int4": (_c_i32, [ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.c_int, _c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]),
    "moe_swiglu_quant": (_c_i32, [ctypes.c_int, _vp, _c_i64, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp]),
    "moe_pack_weight_bf16": (_c_i32, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp]),
    "moe_grouped_gemm_bf16": (_c_i32, [ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.c_int, _c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]),
    "moe_quant_weight_fp4": (_c_i32, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]),
    "moe_pack_weight_fp4": (_c_i32, [_vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]),
    "moe_grouped_gemm_fp8_fp4": (_c_i32, [ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          ctypes.c_int, _c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]),
    "moe_quant_act_int8": (_c_i32, [_vp, _c_i64, ctypes.c_int, _vp, _vp, _vp]),
    "moe_quant_weight_int8": (_c_i32, [_vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]),
    "moe_grouped_gemm_int8": (_c_i32, [ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.c_int, _c_i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]),
    "moe_unpermute_combine": (_c_i32, [_vp, _c_i64, _vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp]),
    "moe_stream_read_words": (ctypes.c_int, []),
    "moe_stream_read": (_c_i32, [_vp, _c_i64, _vp, _vp]),
}


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libmoe.so (once).  Raises ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m int4_weights_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, fn: str):
    if status != 0:
        msg = load().moe_last_error().decode(errors="replace")
        raise MoeError(status, fn, msg)


def _dev(t, name, dtype=None, ndim=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _row_bytes(t) -> int:
    return math.prod(t.shape[1:]) * t.element_size()


def moe_abi_version() -> int:
    return load().moe_abi_version()


def moe_packed_rows_cap(T: int, k: int, E: int, align: int) -> int:
    return int(load().moe_packed_rows_cap(T, k, E, align))


def moe_route_pack_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(load().moe_route_pack_workspace_bytes(T, k, E))


def moe_quant_act(x, q, sf, stream=None):
    """x bf16 [rows, K] -> q uint8 [rows, K] (E4M3 codes), sf float32 [rows, K/128]."""
    _dev(x, "x", torch.bfloat16, 2), _dev(q, "q", torch.uint8, 2), _dev(sf, "sf", torch.float32, 2)
    rows, K = x.shape
    if tuple(q.shape) != (rows, K) or tuple(sf.shape) != (rows, K // 128):
        raise ValueError("moe_quant_act: shape mismatch")
    _check(load().moe_quant_act(_ptr(x), rows, K, _ptr(q), _ptr(sf), _stream(stream)), "moe_quant_act")


def moe_quant_weight_fp8(w, q, sfw, stream=None):
    """w bf16 [E, N, K] -> q uint8 [E, N, K], sfw float32 [E, N/128, K/128]."""
    _dev(w, "w", torch.bfloat16, 3), _dev(q, "q", torch.uint8, 3), _dev(sfw, "sfw", torch.float32, 3)
    E, N, K = w.shape
    if tuple(q.shape) != (E, N, K) or tuple(sfw.shape) != (E, N // 128, K // 128):
        raise ValueError("moe_quant_weight_fp8: shape mismatch")
    _check(load().moe_quant_weight_fp8(_ptr(w), E, N, K, _ptr(q), _ptr(sfw), _stream(stream)),
           "moe_quant_weight_fp8")


def moe_pack_weight_fp8(q, packed, stream=None):
    """q uint8 [E, N, K] (row-major codes) -> packed uint8 [E, N, K] in the fragment order (see include/moe.h)."""
    _dev(q, "q", torch.uint8, 3), _dev(packed, "packed", torch.uint8, 3)
    E, N, K = q.shape
    if tuple(packed.shape) != (E, N, K):
        raise ValueError("moe_pack_weight_fp8: shape mismatch")
    _check(load().moe_pack_weight_fp8(_ptr(q), E, N, K, _ptr(packed), _stream(stream)), "moe_pack_weight_fp8")


def moe_pack_weight_int4(q4, s16, q4_packed, s16_packed, stream=None):
    """q4 uint8 [E, N, K/2] and s16 fp16 [E, N, K/128] (MatMulNBits order) -> the packed orders, same shapes."""
    _dev(q4, "q4", torch.uint8, 3), _dev(q4_packed, "q4_packed", torch.uint8, 3)
    _dev(s16, "s16", torch.float16, 3), _dev(s16_packed, "s16_packed", torch.float16, 3)
    E, N, K2 = q4.shape
    if tuple(q4_packed.shape) != (E, N, K2) or tuple(s16.shape) != (E, N, K2 // 64) or \
            tuple(s16_packed.shape) != (E, N, K2 // 64):
        raise ValueError("moe_pack_weight_int4: shape mismatch")
    _check(load().moe_pack_weight_int4(_ptr(q4), _ptr(s16), E, N, 2 * K2, _ptr(q4_packed), _ptr(s16_packed),
                                       _stream(stream)), "moe_pack_weight_int4")


def moe_quant_weight_int4(w, q4, s16, stream=None):
    """w bf16 [E, N, K] -> q4 uint8 [E, N, K/2], s16 float16 [E, N, K/128]."""
    _dev(w, "w", torch.bfloat16, 3), _dev(q4, "q4", torch.uint8, 3), _dev(s16, "s16", torch.float16, 3)
    E, N, K = w.shape
    if tuple(q4.shape) != (E, N, K // 2) or tuple(s16.shape) != (E, N, K // 128):
        raise ValueError("moe_quant_weight_int4: shape mismatch")
    _check(load().moe_quant_weight_int4(_ptr(w), E, N, K, _ptr(q4), _ptr(s16), _stream(stream)),
           "moe_quant_weight_int4")


def moe_route_pack(topk_ids, E: int, layout: int, align_or_max_m: int, payload, packed, counts, seg_offsets,
                   m_indices, output_index, dev_status, payload2=None, packed2=None, workspace=None, stream=None):
    """See include/moe.h.  payload [T, ...] and packed [rows_cap, ...] are any contiguous tensors;
    their row byte counts are taken from the last dimensions."""
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    for n, t in (("payload", payload), ("packed", packed), ("payload2", payload2), ("packed2", packed2)):
        _dev(t, n)
    for n, t in (("counts", counts), ("seg_offsets", seg_offsets), ("m_indices", m_indices),
                 ("output_index", output_index), ("dev_status", dev_status)):
        _dev(t, n, torch.int32)
    _dev(workspace, "workspace")
    T, k = topk_ids.shape
    rb = _row_bytes(payload)
    rows_cap = packed.shape[0]
    if _row_bytes(packed) != rb:
        raise ValueError("moe_route_pack: payload and packed rows differ in size")
    rb2 = 0
    if payload2 is not None:
        rb2 = _row_bytes(payload2)
        if packed2 is None or packed2.shape[0] != rows_cap or _row_bytes(packed2) != rb2:
            raise ValueError("moe_route_pack: payload2/packed2 mismatch")
    if m_indices.numel() < rows_cap or counts.numel() < E or seg_offsets.numel() < E + 1 or \
            output_index.numel() < T * k:
        raise ValueError("moe_route_pack: output arrays too small")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().moe_route_pack(_ptr(topk_ids), T, k, E, layout, align_or_max_m,
                                 _ptr(payload), rb, _ptr(payload2), rb2, _ptr(packed), _ptr(packed2), rows_cap,
                                 _ptr(counts), _ptr(seg_offsets), _ptr(m_indices), _ptr(output_index),
                                 _ptr(dev_status), _ptr(workspace), ws_bytes, _stream(stream)), "moe_route_pack")


def moe_route_pack_quant(topk_ids, E: int, layout: int, align_or_max_m: int, x, packed_q, packed_sf, counts,
                         seg_offsets, m_indices, output_index, dev_status, workspace=None, stream=None):
    """moe_quant_act + moe_route_pack in one call: x bf16 [T, K] -> packed_q uint8 [rows_cap, K] (E4M3 codes) and
    packed_sf float32 [rows_cap, K/128], plus the routing outputs of moe_route_pack."""
    _dev(topk_ids, "topk_ids", torch.int32, 2), _dev(x, "x", torch.bfloat16, 2)
    _dev(packed_q, "packed_q", torch.uint8, 2), _dev(packed_sf, "packed_sf", torch.float32, 2)
    for n, t in (("counts", counts), ("seg_offsets", seg_offsets), ("m_indices", m_indices),
                 ("output_index", output_index), ("dev_status", dev_status)):
        _dev(t, n, torch.int32)
    _dev(workspace, "workspace")
    T, k = topk_ids.shape
    K = x.shape[1]
    rows_cap = packed_q.shape[0]
    if x.shape[0] != T or packed_q.shape[1] != K or tuple(packed_sf.shape) != (rows_cap, K // 128):
        raise ValueError("moe_route_pack_quant: shape mismatch")
    if m_indices.numel() < rows_cap or counts.numel() < E or seg_offsets.numel() < E + 1 or \
            output_index.numel() < T * k:
        raise ValueError("moe_route_pack_quant: output arrays too small")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().moe_route_pack_quant(_ptr(topk_ids), T, k, E, layout, align_or_max_m, _ptr(x), K, _ptr(packed_q),
                                       _ptr(packed_sf), rows_cap, _ptr(counts), _ptr(seg_offsets), _ptr(m_indices),
                                       _ptr(output_index), _ptr(dev_status), _ptr(workspace), ws_bytes,
                                       _stream(stream)), "moe_route_pack_quant")


def moe_route_pack_noalloc_max_bytes() -> int:
    return int(load().moe_route_pack_noalloc_max_bytes())


def moe_route_pack_noalloc(topk_ids, E: int, layout: int, align_or_max_m: int, payload, packed, counts, seg_offsets,
                           m_indices, output_index, dev_status, payload2=None, packed2=None, stream=None):
    """moe_route_pack without a workspace (the library's fixed device scratch; see include/moe.h)."""
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    for n, t in (("payload", payload), ("packed", packed), ("payload2", payload2), ("packed2", packed2)):
        _dev(t, n)
    for n, t in (("counts", counts), ("seg_offsets", seg_offsets), ("m_indices", m_indices),
                 ("output_index", output_index), ("dev_status", dev_status)):
        _dev(t, n, torch.int32)
    T, k = topk_ids.shape
    rb = _row_bytes(payload)
    rows_cap = packed.shape[0]
    if _row_bytes(packed) != rb:
        raise ValueError("moe_route_pack_noalloc: payload and packed rows differ in size")
    rb2 = 0
    if payload2 is not None:
        rb2 = _row_bytes(payload2)
        if packed2 is None or packed2.shape[0] != rows_cap or _row_bytes(packed2) != rb2:
            raise ValueError("moe_route_pack_noalloc: payload2/packed2 mismatch")
    if m_indices.numel() < rows_cap or counts.numel() < E or seg_offsets.numel() < E + 1 or \
            output_index.numel() < T * k:
        raise ValueError("moe_route_pack_noalloc: output arrays too small")
    _check(load().moe_route_pack_noalloc(_ptr(topk_ids), T, k, E, layout, align_or_max_m,
                                         _ptr(payload), rb, _ptr(payload2), rb2, _ptr(packed), _ptr(packed2),
                                         rows_cap, _ptr(counts), _ptr(seg_offsets), _ptr(m_indices),
                                         _ptr(output_index), _ptr(dev_status), _stream(stream)),
           "moe_route_pack_noalloc")


def _gemm_sizes(fn, layout, E, rows_cap_or_max_m, counts, seg_offsets, sizes):
    layout &= ~WEIGHTS_PACKED
    rows = E * rows_cap_or_max_m if layout == LAYOUT_MASKED else rows_cap_or_max_m
    if counts.numel() < E or (layout == LAYOUT_CONTIGUOUS and (seg_offsets is None or seg_offsets.numel() < E)):
        raise ValueError(f"{fn}: counts/seg_offsets too small")
    for name, t, need in sizes(rows):
        if t.numel() < need:
            raise ValueError(f"{fn}: {name} has {t.numel()} elements, needs {need}")


def moe_grouped_gemm_fp8(layout: int, A, SFA, W, SFW, D, counts, seg_offsets, E: int, rows_cap_or_max_m: int,
                         N: int, K: int, expected_m: int = 0, stream=None):
    _dev(A, "A", torch.uint8), _dev(SFA, "SFA", torch.float32), _dev(W, "W", torch.uint8)
    _dev(SFW, "SFW", torch.float32), _dev(D, "D", torch.bfloat16), _dev(counts, "counts", torch.int32)
    _dev(seg_offsets, "seg_offsets", torch.int32)
    _gemm_sizes("moe_grouped_gemm_fp8", layout, E, rows_cap_or_max_m, counts, seg_offsets,
                lambda rows: (("A", A, rows * K), ("SFA", SFA, rows * (K // 128)), ("W", W, E * N * K),
                              ("SFW", SFW, E * (N // 128) * (K // 128)), ("D", D, rows * N)))
    _check(load().moe_grouped_gemm_fp8(layout, _ptr(A), _ptr(SFA), _ptr(W), _ptr(SFW), _ptr(D), _ptr(counts),
                                       _ptr(seg_offsets), E, rows_cap_or_max_m, N, K, expected_m, _stream(stream)),
           "moe_grouped_gemm_fp8")


def moe_grouped_gemm_fp8_swiglu(layout: int, A, SFA, W, SFW, Q, SQ, counts, seg_offsets, E: int,
                                rows_cap_or_max_m: int, I: int, K: int, expected_m: int = 0, stream=None):
    """The up-projection (W [E, 2I, K]: gate rows, then up rows) with SwiGLU and the 1x128 requantisation:
    Q uint8 [rows, I] E4M3 codes, SQ float32 [rows, I/128] (see include/moe.h)."""
    _dev(A, "A", torch.uint8), _dev(SFA, "SFA", torch.float32), _dev(W, "W", torch.uint8)
    _dev(SFW, "SFW", torch.float32), _dev(Q, "Q", torch.uint8), _dev(SQ, "SQ", torch.float32)
    _dev(counts, "counts", torch.int32), _dev(seg_offsets, "seg_offsets", torch.int32)
    _gemm_sizes("moe_grouped_gemm_fp8_swiglu", layout, E, rows_cap_or_max_m, counts, seg_offsets,
                lambda rows: (("A", A, rows * K), ("SFA", SFA, rows * (K // 128)), ("W", W, E * 2 * I * K),
                              ("SFW", SFW, E * (2 * I // 128) * (K // 128)), ("Q", Q, rows * I),
                              ("SQ", SQ, rows * (I // 128))))
    _check(load().moe_grouped_gemm_fp8_swiglu(layout, _ptr(A), _ptr(SFA), _ptr(W), _ptr(SFW), _ptr(Q), _ptr(SQ),
                                              _ptr(counts), _ptr(seg_offsets), E, rows_cap_or_max_m, I, K,
                                              expected_m, _stream(stream)),
           "moe_grouped_gemm_fp8_swiglu")


def moe_grouped_gemm_int4(layout: int, A, W4, S16, D, counts, seg_offsets, E: int, rows_cap_or_max_m: int,
                          N: int, K: int, expected_m: int = 0, stream=None):
    _dev(A, "A", torch.bfloat16), _dev(W4, "W4", torch.uint8), _dev(S16, "S16", torch.float16)
    _dev(D, "D", torch.bfloat16), _dev(counts, "counts", torch.int32), _dev(seg_offsets, "seg_offsets", torch.int32)
    _gemm_sizes("moe_grouped_gemm_int4", layout, E, rows_cap_or_max_m, counts, seg_offsets,
                lambda rows: (("A", A, rows * K), ("W4", W4, E * N * (K // 2)), ("S16", S16, E * N * (K // 128)),
                              ("D", D, rows * N)))
    _check(load().moe_grouped_gemm_int4(layout, _ptr(A), _ptr(W4), _ptr(S16), _ptr(D), _ptr(counts),
                                        _ptr(seg_offsets), E, rows_cap_or_max_m, N, K, expected_m, _stream(stream)),
           "moe_grouped_gemm_int4")


def moe_pack_weight_bf16(w, packed, stream=None):
    """w bf16 [E, N, K] -> packed bf16 [E, N, K] in the fragment order (see include/moe.h)."""
    _dev(w, "w", torch.bfloat16, 3), _dev(packed, "packed", torch.bfloat16, 3)
    E, N, K = w.shape
    if tuple(packed.shape) != (E, N, K):
        raise ValueError("moe_pack_weight_bf16: shape mismatch")
    _check(load().moe_pack_weight_bf16(_ptr(w), E, N, K, _ptr(packed), _stream(stream)), "moe_pack_weight_bf16")


def moe_grouped_gemm_bf16(layout: int, A, W, D, counts, seg_offsets, E: int, rows_cap_or_max_m: int, N: int, K: int,
                          expected_m: int = 0, stream=None):
    _dev(A, "A", torch.bfloat16), _dev(W, "W", torch.bfloat16), _dev(D, "D", torch.bfloat16)
    _dev(counts, "counts", torch.int32), _dev(seg_offsets, "seg_offsets", torch.int32)
    _gemm_sizes("moe_grouped_gemm_bf16", layout, E, rows_cap_or_max_m, counts, seg_offsets,
                lambda rows: (("A", A, rows * K), ("W", W, E * N * K), ("D", D, rows * N)))
    _check(load().moe_grouped_gemm_bf16(layout, _ptr(A), _ptr(W), _ptr(D), _ptr(counts), _ptr(seg_offsets), E,
                                        rows_cap_or_max_m, N, K, expected_m, _stream(stream)),
           "moe_grouped_gemm_bf16")


def moe_quant_weight_fp4(w, w4, sw, stream=None):
    """w bf16 [E, N, K] -> w4 uint8 [E, N, K/2] (E2M1 pairs), sw uint8 [E, N, K/32] (E8M0 scales)."""
    _dev(w, "w", torch.bfloat16, 3), _dev(w4, "w4", torch.uint8, 3), _dev(sw, "sw", torch.uint8, 3)
    E, N, K = w.shape
    if tuple(w4.shape) != (E, N, K // 2) or tuple(sw.shape) != (E, N, K // 32):
        raise ValueError("moe_quant_weight_fp4: shape mismatch")
    _check(load().moe_quant_weight_fp4(_ptr(w), E, N, K, _ptr(w4), _ptr(sw), _stream(stream)), "moe_quant_weight_fp4")


def moe_pack_weight_fp4(w4, sw, w4_packed, sw_packed, stream=None):
    """MXFP4 codes uint8 [E, N, K/2] and scales uint8 [E, N, K/32] -> the packed orders, same shapes."""
    _dev(w4, "w4", torch.uint8, 3), _dev(sw, "sw", torch.uint8, 3)
    _dev(w4_packed, "w4_packed", torch.uint8, 3), _dev(sw_packed, "sw_packed", torch.uint8, 3)
    E, N, K2 = w4.shape
    if tuple(w4_packed.shape) != (E, N, K2) or tuple(sw.shape) != (E, N, K2 // 16) or \
            tuple(sw_packed.shape) != (E, N, K2 // 16):
        raise ValueError("moe_pack_weight_fp4: shape mismatch")
    _check(load().moe_pack_weight_fp4(_ptr(w4), _ptr(sw), E, N, 2 * K2, _ptr(w4_packed), _ptr(sw_packed),
                                      _stream(stream)), "moe_pack_weight_fp4")


def moe_grouped_gemm_fp8_fp4(layout: int, A, SFA, W4, SW, D, counts, seg_offsets, E: int, rows_cap_or_max_m: int,
                             N: int, K: int, expected_m: int = 0, stream=None):
    _dev(A, "A", torch.uint8), _dev(SFA, "SFA", torch.float32), _dev(W4, "W4", torch.uint8)
    _dev(SW, "SW", torch.uint8), _dev(D, "D", torch.bfloat16), _dev(counts, "counts", torch.int32)
    _dev(seg_offsets, "seg_offsets", torch.int32)
    _gemm_sizes("moe_grouped_gemm_fp8_fp4", layout, E, rows_cap_or_max_m, counts, seg_offsets,
                lambda rows: (("A", A, rows * K), ("SFA", SFA, rows * (K // 128)), ("W4", W4, E * N * (K // 2)),
                              ("SW", SW, E * N * (K // 32)), ("D", D, rows * N)))
    _check(load().moe_grouped_gemm_fp8_fp4(layout, _ptr(A), _ptr(SFA), _ptr(W4), _ptr(SW), _ptr(D), _ptr(counts),
                                           _ptr(seg_offsets), E, rows_cap_or_max_m, N, K, expected_m,
                                           _stream(stream)), "moe_grouped_gemm_fp8_fp4")


def moe_quant_act_int8(x, q, s, stream=None):
    """x bf16 [rows, K] -> q int8 [rows, K], s float32 [rows, K/128] (INT8 (1, 1, 128), symmetric amax / 127)."""
    _dev(x, "x", torch.bfloat16, 2), _dev(q, "q", torch.int8, 2), _dev(s, "s", torch.float32, 2)
    rows, K = x.shape
    if tuple(q.shape) != (rows, K) or tuple(s.shape) != (rows, K // 128):
        raise ValueError("moe_quant_act_int8: shape mismatch")
    _check(load().moe_quant_act_int8(_ptr(x), rows, K, _ptr(q), _ptr(s), _stream(stream)), "moe_quant_act_int8")


def moe_quant_weight_int8(w, q, sw, stream=None):
    """w bf16 [E, N, K] -> q int8 [E, N, K], sw float32 [E, K/128, N] (per-channel scales, K-block-major)."""
    _dev(w, "w", torch.bfloat16, 3), _dev(q, "q", torch.int8, 3), _dev(sw, "sw", torch.float32, 3)
    E, N, K = w.shape
    if tuple(q.shape) != (E, N, K) or tuple(sw.shape) != (E, K // 128, N):
        raise ValueError("moe_quant_weight_int8: shape mismatch")
    _check(load().moe_quant_weight_int8(_ptr(w), E, N, K, _ptr(q), _ptr(sw), _stream(stream)),
           "moe_quant_weight_int8")


def moe_grouped_gemm_int8(layout: int, A, SA, W, SW, D, counts, seg_offsets, E: int, rows_cap_or_max_m: int,
                          N: int, K: int, expected_m: int = 0, stream=None):
    """int8 A [rows, K] with SA [rows, K/128] x int8 W [E, N, K] (or moe_pack_weight_fp8's order) with
    SW [E, K/128, N] -> D bf16 [rows, N]."""
    _dev(A, "A", torch.int8), _dev(SA, "SA", torch.float32), _dev(W, "W")
    _dev(SW, "SW", torch.float32), _dev(D, "D", torch.bfloat16), _dev(counts, "counts", torch.int32)
    _dev(seg_offsets, "seg_offsets", torch.int32)
    if W.dtype not in (torch.int8, torch.uint8):
        raise ValueError("W must be int8 (or uint8 from moe_pack_weight_fp8)")
    _gemm_sizes("moe_grouped_gemm_int8", layout, E, rows_cap_or_max_m, counts, seg_offsets,
                lambda rows: (("A", A, rows * K), ("SA", SA, rows * (K // 128)), ("W", W, E * N * K),
                              ("SW", SW, E * (K // 128) * N), ("D", D, rows * N)))
    _check(load().moe_grouped_gemm_int8(layout, _ptr(A), _ptr(SA), _ptr(W), _ptr(SW), _ptr(D), _ptr(counts),
                                        _ptr(seg_offsets), E, rows_cap_or_max_m, N, K, expected_m, _stream(stream)),
           "moe_grouped_gemm_int8")


def moe_swiglu_quant(layout: int, gate_up, rows_cap_or_max_m: int, counts, seg_offsets, E: int, q, sf,
                     stream=None):
    """gate_up bf16 [rows, 2I] -> q uint8 [rows, I] (E4M3 codes of silu(gate)*up), sf float32 [rows, I/128]."""
    _dev(gate_up, "gate_up", torch.bfloat16), _dev(q, "q", torch.uint8), _dev(sf, "sf", torch.float32)
    _dev(counts, "counts", torch.int32), _dev(seg_offsets, "seg_offsets", torch.int32)
    I = gate_up.shape[-1] // 2
    rows = E * rows_cap_or_max_m if layout == LAYOUT_MASKED else rows_cap_or_max_m
    if gate_up.numel() < rows * 2 * I or q.numel() < rows * I or sf.numel() < rows * (I // 128) or \
            counts.numel() < E or (layout == LAYOUT_CONTIGUOUS and (seg_offsets is None or seg_offsets.numel() < E)):
        raise ValueError("moe_swiglu_quant: buffers too small")
    _check(load().moe_swiglu_quant(layout, _ptr(gate_up), rows_cap_or_max_m, I, _ptr(counts), _ptr(seg_offsets), E,
                                   _ptr(q), _ptr(sf), _stream(stream)), "moe_swiglu_quant")


def moe_unpermute_combine(Y, output_index, topk_weights, Z, stream=None):
    """Y bf16 [y_rows, N], output_index int32 [T, k], topk_weights float32 [T, k] -> Z bf16 [T, N]."""
    _dev(Y, "Y", torch.bfloat16, 2), _dev(output_index, "output_index", torch.int32, 2)
    _dev(topk_weights, "topk_weights", torch.float32, 2), _dev(Z, "Z", torch.bfloat16, 2)
    T, k = output_index.shape
    N = Z.shape[1]
    if Y.shape[1] != N or Z.shape[0] != T or tuple(topk_weights.shape) != (T, k):
        raise ValueError("moe_unpermute_combine: shape mismatch")
    _check(load().moe_unpermute_combine(_ptr(Y), Y.shape[0], _ptr(output_index), _ptr(topk_weights), T, k, N,
                                        _ptr(Z), _stream(stream)), "moe_unpermute_combine")


def moe_stream_read_words() -> int:
    """Words moe_stream_read writes (one per workgroup of its grid)."""
    return int(load().moe_stream_read_words())


def moe_stream_read(buf, out, stream=None):
    """Read every byte of the device tensor buf once (a measurement helper); out: int32 [moe_stream_read_words()]
    receives the XOR fold of the words read."""
    if buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("moe_stream_read: buf must be a contiguous device tensor")
    _dev(out, "out", torch.int32, 1)
    nbytes = buf.numel() * buf.element_size()
    if out.numel() < moe_stream_read_words():
        raise ValueError("moe_stream_read: out too small")
    _check(load().moe_stream_read(_ptr(buf), nbytes, _ptr(out), _stream(stream)), "moe_stream_read")
