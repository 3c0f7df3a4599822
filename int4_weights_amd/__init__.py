"""MoE grouped GEMM on gfx950 (MI355X): FP8 block-scaled, 4-bit weight-only, FP4, INT8 and BF16.

The compute path is libmoe.so (hand-written HIP kernels behind the C ABI in
include/moe.h); this package is its thin Python binding.  Build the library
with ``python -m int4_weights_amd.build``; calls raise if it is missing.
"""

from ._lib import (  # noqa: F401
    DEV_CAPACITY,
    DEV_ID_RANGE,
    LAYOUT_CONTIGUOUS,
    LAYOUT_MASKED,
    LIB_PATH,
    SIGNATURES,
    WEIGHTS_PACKED,
    MoeError,
    load,
    moe_abi_version,
    moe_grouped_gemm_bf16,
    moe_grouped_gemm_fp8,
    moe_grouped_gemm_fp8_fp4,
    moe_grouped_gemm_fp8_swiglu,
    moe_grouped_gemm_int4,
    moe_grouped_gemm_int8,
    moe_pack_weight_bf16,
    moe_pack_weight_fp4,
    moe_pack_weight_fp8,
    moe_pack_weight_int4,
    moe_packed_rows_cap,
    moe_quant_act,
    moe_quant_act_int8,
    moe_quant_weight_fp4,
    moe_quant_weight_fp8,
    moe_quant_weight_int4,
    moe_quant_weight_int8,
    moe_route_pack,
    moe_route_pack_noalloc,
    moe_route_pack_quant,
    moe_route_pack_noalloc_max_bytes,
    moe_route_pack_workspace_bytes,
    moe_swiglu_quant,
    moe_stream_read,
    moe_stream_read_words,
    moe_unpermute_combine,
)
