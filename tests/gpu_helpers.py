"""Shared helpers for the GPU parity tests (tests import the oracle; the product never does)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
import oracle

DEV = "cuda:0"


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()  # fail loudly if the HIP library is missing


def u16(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16/fp16 tensor (host numpy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_from_u16(a: np.ndarray, device=DEV) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def fp8_quant_gpu(x: torch.Tensor):
    rows, K = x.shape
    q = torch.empty(rows, K, dtype=torch.uint8, device=x.device)
    sf = torch.empty(rows, K // 128, dtype=torch.float32, device=x.device)
    moe.moe_quant_act(x, q, sf)
    return q, sf


def fp8_quant_weight_gpu(w: torch.Tensor):
    E, N, K = w.shape
    q = torch.empty(E, N, K, dtype=torch.uint8, device=w.device)
    sfw = torch.empty(E, N // 128, K // 128, dtype=torch.float32, device=w.device)
    moe.moe_quant_weight_fp8(w, q, sfw)
    return q, sfw


def int4_quant_weight_gpu(w: torch.Tensor):
    E, N, K = w.shape
    q4 = torch.empty(E, N, K // 2, dtype=torch.uint8, device=w.device)
    s16 = torch.empty(E, N, K // 128, dtype=torch.float16, device=w.device)
    moe.moe_quant_weight_int4(w, q4, s16)
    return q4, s16


class Routed:
    """Outputs of one moe_route_pack call (device tensors)."""

    def __init__(self, ids, E, layout, am, payload, payload2=None, rows_cap=None, fill=None):
        T, k = ids.shape
        self.T, self.k, self.E = T, k, E
        self.layout = layout
        self.am = am
        if rows_cap is None:
            rows_cap = moe.moe_packed_rows_cap(T, k, E, am) if layout == moe.LAYOUT_CONTIGUOUS else E * am
        self.rows_cap = rows_cap
        dev = payload.device
        self.packed = torch.empty((rows_cap,) + tuple(payload.shape[1:]), dtype=payload.dtype, device=dev)
        if fill is not None:
            self.packed.view(torch.uint8).fill_(fill)
        self.packed2 = None
        if payload2 is not None:
            self.packed2 = torch.empty((rows_cap,) + tuple(payload2.shape[1:]), dtype=payload2.dtype, device=dev)
            if fill is not None:
                self.packed2.view(torch.uint8).fill_(fill)
        self.counts = torch.full((E,), -7, dtype=torch.int32, device=dev)
        self.seg_offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
        self.m_indices = torch.full((rows_cap,), -7, dtype=torch.int32, device=dev)
        self.output_index = torch.full((T, k), -7, dtype=torch.int32, device=dev)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=dev)
        wsb = moe.moe_route_pack_workspace_bytes(T, k, E)
        self.workspace = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev) if wsb > 0 else None
        moe.moe_route_pack(ids, E, layout, am, payload, self.packed, self.counts, self.seg_offsets, self.m_indices,
                           self.output_index, self.dev_status, payload2=payload2, packed2=self.packed2,
                           workspace=self.workspace)


def oracle_route(ids: torch.Tensor, E: int, layout: int, am: int, rows_cap: int):
    lay = "contiguous" if layout == moe.LAYOUT_CONTIGUOUS else "masked"
    kw = {"align": am} if lay == "contiguous" else {"max_m": am}
    return oracle.route(ids.cpu().numpy(), E, lay, rows_cap=rows_cap, **kw)


def valid_rows(counts: np.ndarray, starts: np.ndarray) -> np.ndarray:
    rows = [np.arange(int(s), int(s) + int(c)) for c, s in zip(counts, starts[: len(counts)]) if c > 0]
    return np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)


def gemm_tolerance_check(got: np.ndarray, ref: np.ndarray, bar: float):
    """The path's bar: diff < bar and |err| <= 2e-2*|ref| + 1e-2*rms(ref) per element."""
    d = oracle.calc_diff(got, ref)
    ex = oracle.elementwise_excess(got, ref)
    assert d < bar, f"calc_diff {d:.3e} >= {bar}"
    assert ex <= 0.0, f"per-element bound exceeded by {ex:.3e}"
    return d
