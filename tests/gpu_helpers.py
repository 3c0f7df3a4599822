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


# ------------------------------------------------------------------ SwiGLU --
def _e4m3_midpoints():
    """Sorted float64 midpoints between consecutive non-negative E4M3 values (0 .. 448)."""
    tab = oracle.e4m3_decode_table()[:127]
    return (tab[:-1] + tab[1:]) / 2.0


_MID = _e4m3_midpoints()


def _near_midpoint(v, rel=1e-6):
    a = np.abs(v)
    i = np.clip(np.searchsorted(_MID, a), 1, len(_MID) - 1)
    d = np.minimum(np.abs(a - _MID[i - 1]), np.abs(a - _MID[i]))
    return d <= rel * np.maximum(a, 2.0 ** -9)


def check_swiglu_quant(gu_bits, q, sf, valid, sent_q, sent_sf, rare=1e-4):
    """GPU SwiGLU + 1x128 requantisation (codes q, scales sf over all rows) of the bf16 gate/up rows gu_bits
    (gate columns, then up columns; the valid rows only) against the oracle.

    The GPU evaluates h = silu(gate) * up in fp32 (a few fp32 ulps from the exact value) and the oracle in
    float64, so a code or a scale can differ only where the float64 value lies within that error of a rounding
    boundary of the E4M3 grid or of the power-of-two scale rule.  Required:
      * every scale a power of two, and equal to the oracle's unless the block's float64 amax is within 1e-6
        (relative) of a boundary 448 * 2^k, or below the fp32 normal range (zero codes either way);
      * every code equal to the oracle's unless the block's scale differs or the float64 scaled value is within
        1e-6 (relative) of an E4M3 rounding midpoint -- and such exceptions rare (at most a fraction `rare`);
      * every dequantised value within the E4M3 rounding bound of the float64 h;
      * rows outside the segments untouched (still sent_q / sent_sf).
    Returns the number of code exceptions."""
    I = gu_bits.shape[1] // 2
    assert (q[~valid] == sent_q).all() and (sf[~valid] == sent_sf).all(), "rows outside the segments were written"
    gu = oracle.bf16_bits_to_f64(gu_bits)
    h = oracle.swiglu(gu)
    qo, so = oracle.quant_act_values(h)
    qg, sg = q[valid], sf[valid]
    bits = sg.view(np.uint32)
    assert ((bits & 0x807FFFFF) == 0).all() and (bits != 0).all(), "scales must be powers of two"
    nb = I // 128
    amax = np.abs(h.reshape(-1, nb, 128)).max(axis=2)
    ratio = amax / 448.0
    near_scale = (ratio > 0) & (np.abs(ratio / np.exp2(np.round(np.log2(np.maximum(ratio, 1e-300)))) - 1.0) <= 1e-6)
    # a block whose float64 amax lies below the fp32 normal range underflows to 0 in fp32 (scale 1, zero codes)
    # while float64 keeps a tiny value (scale 2^-126, zero codes): the same zeros, encoded with another scale
    tiny = amax < 2.0 ** -120
    scale_ok = (sg == so) | near_scale | tiny
    assert scale_ok.all(), f"{int((~scale_ok).sum())} block scales differ away from a boundary"
    same_scale = np.repeat(sg == so, 128, axis=1)
    scaled = h / np.repeat(so.astype(np.float64), 128, axis=1)
    code_ok = (qg == qo) | ~same_scale | _near_midpoint(scaled)
    assert code_ok.all(), f"{int((~code_ok).sum())} codes differ away from a rounding midpoint"
    exceptions = int(((qg != qo) & same_scale).sum())
    assert exceptions <= max(2, int(qg.size * rare)), f"{exceptions} of {qg.size} codes differ"
    deq = oracle.dequant_act(qg, sg)
    s = np.repeat(sg.astype(np.float64), 128, axis=1)
    assert (np.abs(deq - h) <= np.maximum(2.0 ** -4 * np.abs(h), 2.0 ** -10 * s) * (1 + 1e-5) + 1e-30).all()
    return exceptions
