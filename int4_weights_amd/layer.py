"""MoE expert layer built on the libmoe entry points.

One forward pass is the data flow of rainlin, "GEMM 执行方式", sec. 4.6:
quantise tokens -> route and pack -> grouped GEMM -> weighted combine, on one
stream with no host synchronisation (the first two steps can run as one call
that quantises while it packs).  Buffers are allocated
once, for a maximum token count, so a forward allocates nothing.
"""

from __future__ import annotations

import torch

from . import _lib as L


class MoeFP8Layer:
    """FP8 block-scaled expert GEMM (1x128 activation scales, 128x128 weight scales)."""

    def __init__(self, w_codes: torch.Tensor, sfw: torch.Tensor, topk: int, max_tokens: int,
                 layout: int = L.LAYOUT_CONTIGUOUS, align_or_max_m: int = 128, expected_m: int = 0,
                 weights_packed: bool = False):
        """weights_packed: w_codes (and any weights passed to gemm()) are in moe_pack_weight_fp8 order."""
        E, N, K = w_codes.shape
        self.wflag = L.WEIGHTS_PACKED if weights_packed else 0
        self.E, self.N, self.K, self.topk = E, N, K, topk
        self.w, self.sfw = w_codes, sfw
        self.layout, self.am = layout, align_or_max_m
        self.expected_m = expected_m
        dev = w_codes.device
        self.max_tokens = max_tokens
        if layout == L.LAYOUT_CONTIGUOUS:
            self.rows_cap = L.moe_packed_rows_cap(max_tokens, topk, E, align_or_max_m)
        else:
            self.rows_cap = E * align_or_max_m
        self.q = torch.empty(max_tokens, K, dtype=torch.uint8, device=dev)
        self.sf = torch.empty(max_tokens, K // 128, dtype=torch.float32, device=dev)
        self.packed = torch.empty(self.rows_cap, K, dtype=torch.uint8, device=dev)
        self.packed_sf = torch.empty(self.rows_cap, K // 128, dtype=torch.float32, device=dev)
        self.counts = torch.zeros(E, dtype=torch.int32, device=dev)
        self.seg_offsets = torch.zeros(E + 1, dtype=torch.int32, device=dev)
        self.m_indices = torch.empty(self.rows_cap, dtype=torch.int32, device=dev)
        self.output_index = torch.empty(max_tokens, topk, dtype=torch.int32, device=dev)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=dev)
        wsb = L.moe_route_pack_workspace_bytes(max_tokens, topk, E)
        self.workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        self.D = torch.empty(self.rows_cap, N, dtype=torch.bfloat16, device=dev)
        self.Z = torch.empty(max_tokens, N, dtype=torch.bfloat16, device=dev)

    def _views(self, T):
        return self.q[:T], self.sf[:T], self.output_index[:T], self.Z[:T]

    def quant(self, x):
        q, sf, _, _ = self._views(x.shape[0])
        L.moe_quant_act(x, q, sf)

    def route(self, topk_ids):
        T = topk_ids.shape[0]
        q, sf, oi, _ = self._views(T)
        rows = L.moe_packed_rows_cap(T, self.topk, self.E, self.am) if self.layout == L.LAYOUT_CONTIGUOUS \
            else self.rows_cap
        L.moe_route_pack(topk_ids, self.E, self.layout, self.am, q, self.packed[:rows], self.counts,
                         self.seg_offsets, self.m_indices[:rows], oi, self.dev_status, payload2=sf,
                         packed2=self.packed_sf[:rows], workspace=self.workspace)

    def quant_route(self, x, topk_ids):
        """quant() and route() in one launch sequence (moe_route_pack_quant): the packed codes and scales are the
        same bits, each token row is quantised once, and the token-order codes (self.q, self.sf) are not written."""
        T = topk_ids.shape[0]
        _, _, oi, _ = self._views(T)
        rows = L.moe_packed_rows_cap(T, self.topk, self.E, self.am) if self.layout == L.LAYOUT_CONTIGUOUS \
            else self.rows_cap
        L.moe_route_pack_quant(topk_ids, self.E, self.layout, self.am, x, self.packed[:rows],
                               self.packed_sf[:rows], self.counts, self.seg_offsets, self.m_indices[:rows], oi,
                               self.dev_status, workspace=self.workspace)

    def gemm(self, A=None, SFA=None, D=None, w=None, sfw=None, N=None, K=None):
        """Grouped GEMM on the packed rows (defaults: this layer's buffers and weights)."""
        A = self.packed if A is None else A
        SFA = self.packed_sf if SFA is None else SFA
        D = self.D if D is None else D
        w = self.w if w is None else w
        sfw = self.sfw if sfw is None else sfw
        N = self.N if N is None else N
        K = self.K if K is None else K
        am = self.am if self.layout == L.LAYOUT_MASKED else self.rows_cap
        L.moe_grouped_gemm_fp8(self.layout | self.wflag, A, SFA, w, sfw, D, self.counts, self.seg_offsets, self.E,
                               am, N, K, self.expected_m)

    def swiglu_quant(self, q, sf, D=None):
        """silu(gate) * up of the up-projection output D (default: this layer's), requantised into the
        down-projection's FP8 codes q [rows, N/2] and 1x128 scales sf [rows, N/256]."""
        D = self.D if D is None else D
        am = self.am if self.layout == L.LAYOUT_MASKED else self.rows_cap
        L.moe_swiglu_quant(self.layout, D, am, self.counts, self.seg_offsets, self.E, q, sf)

    def gemm_swiglu(self, q, sf):
        """The up-projection on the packed rows with SwiGLU and the requantisation fused (this layer's weights
        are the up-projection's, N = 2I): codes q [rows, N/2] and 1x128 scales sf [rows, N/256], the same bits
        as gemm() followed by swiglu_quant(), without the bf16 output D."""
        am = self.am if self.layout == L.LAYOUT_MASKED else self.rows_cap
        L.moe_grouped_gemm_fp8_swiglu(self.layout | self.wflag, self.packed, self.packed_sf, self.w, self.sfw, q, sf,
                                      self.counts, self.seg_offsets, self.E, am, self.N // 2, self.K,
                                      self.expected_m)

    def combine(self, topk_weights, D=None, Z=None):
        """Weighted combine of packed rows D (default: this layer's GEMM output) into Z [T, D.shape[1]]."""
        T = topk_weights.shape[0]
        _, _, oi, Zl = self._views(T)
        D = self.D if D is None else D
        if Z is None:
            if D.shape[1] != self.N:
                raise ValueError("pass Z when D is not [rows, N]")
            Z = Zl
        L.moe_unpermute_combine(D, oi, topk_weights, Z)
        return Z

    def forward(self, x, topk_ids, topk_weights, fused_quant=False):
        """fused_quant: quantise while packing (quant_route) instead of quant() then route()."""
        if fused_quant:
            self.quant_route(x, topk_ids)
        else:
            self.quant(x)
            self.route(topk_ids)
        self.gemm()
        return self.combine(topk_weights)


class MoeInt4Layer:
    """4-bit weight-only expert GEMM (group 128, fp16 scales, zero point 8), bf16 activations."""

    def __init__(self, w_q4: torch.Tensor, s16: torch.Tensor, topk: int, max_tokens: int,
                 layout: int = L.LAYOUT_MASKED, align_or_max_m: int = 16, expected_m: int = 0,
                 weights_packed: bool = False):
        """weights_packed: w_q4 is in the order written by moe_pack_weight_int4."""
        E, N, K2 = w_q4.shape
        K = K2 * 2
        self.E, self.N, self.K, self.topk = E, N, K, topk
        self.w, self.s16 = w_q4, s16
        self.wflag = L.WEIGHTS_PACKED if weights_packed else 0
        self.layout, self.am, self.expected_m = layout, align_or_max_m, expected_m
        dev = w_q4.device
        if layout == L.LAYOUT_CONTIGUOUS:
            self.rows_cap = L.moe_packed_rows_cap(max_tokens, topk, E, align_or_max_m)
        else:
            self.rows_cap = E * align_or_max_m
        self.packed = torch.empty(self.rows_cap, K, dtype=torch.bfloat16, device=dev)
        self.counts = torch.zeros(E, dtype=torch.int32, device=dev)
        self.seg_offsets = torch.zeros(E + 1, dtype=torch.int32, device=dev)
        self.m_indices = torch.empty(self.rows_cap, dtype=torch.int32, device=dev)
        self.output_index = torch.empty(max_tokens, topk, dtype=torch.int32, device=dev)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=dev)
        wsb = L.moe_route_pack_workspace_bytes(max_tokens, topk, E)
        self.workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        self.D = torch.empty(self.rows_cap, N, dtype=torch.bfloat16, device=dev)
        self.Z = torch.empty(max_tokens, N, dtype=torch.bfloat16, device=dev)

    def route(self, x, topk_ids):
        T = topk_ids.shape[0]
        rows = L.moe_packed_rows_cap(T, self.topk, self.E, self.am) if self.layout == L.LAYOUT_CONTIGUOUS \
            else self.rows_cap
        L.moe_route_pack(topk_ids, self.E, self.layout, self.am, x, self.packed[:rows], self.counts,
                         self.seg_offsets, self.m_indices[:rows], self.output_index[:T], self.dev_status,
                         workspace=self.workspace)

    def gemm(self, w=None, s16=None):
        w = self.w if w is None else w
        s16 = self.s16 if s16 is None else s16
        am = self.am if self.layout == L.LAYOUT_MASKED else self.rows_cap
        L.moe_grouped_gemm_int4(self.layout | self.wflag, self.packed, w, s16, self.D, self.counts, self.seg_offsets,
                                self.E, am, self.N, self.K, self.expected_m)

    def combine(self, topk_weights):
        T = topk_weights.shape[0]
        L.moe_unpermute_combine(self.D, self.output_index[:T], topk_weights, self.Z[:T])
        return self.Z[:T]

    def forward(self, x, topk_ids, topk_weights):
        self.route(x, topk_ids)
        self.gemm()
        return self.combine(topk_weights)
