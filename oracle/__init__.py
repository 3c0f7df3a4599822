"""CPU oracle for the MoE grouped-GEMM path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports it and never falls back to it.

It is a plain, slow, obviously correct NumPy implementation of what the path
computes, in float64 unless a step turns a floating-point value into an
integer code (then it uses the precision the step is defined in and says so).
It shares no code with the HIP path.

Sources (the five pages the method is described on):
  [GEMM-modes]  rainlin, "GEMM 执行方式" (GEMM execution modes): grouped GEMM
                definition (sec. 4.1), top-2 routing (4.2), packed layout (4.3),
                expert compute and combine (4.4), 128-row alignment and the
                scatter/GEMM/gather flow (4.6).
  [AsymGEMM]    bytedance-iaas "AsymGEMM" README: contiguous and masked token
                layouts ("Token Layout Protocols"), FP8 grouped-GEMM API with
                (data, scale) operands and block recipes ("API Reference").
  [DG-FP8]      nxmr.cn article on DeepGEMM's FP8 precision: E4M3 format and
                range, the (gran_m, gran_n, gran_k) scale recipe, power-of-two
                scale factors ("补偿机制一"), test thresholds ("精度与吞吐的平衡点").
  [MatMulNBits] ONNX Runtime "MatMulNBits -- CUDA Operator Documentation":
                4-bit weight format and zero point 8 (sec. 2 "Weight Format").
  [CuTeDSL]     Perplexity, "CuTeDSL bei Perplexity": MoE dispatch (count per
                expert, unique index within the expert, copy into padded
                buffers) and combine (weighted accumulation); activation
                kernels in the MoE kernel library.

Parity status of every function is listed in its docstring ("pinned by ...").
"""

from .formats import (
    E4M3_MAX,
    e4m3_value,
    e4m3_decode_table,
    e4m3_encode,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    f64_to_bf16_bits_normal,
    fp16_bits_to_f64,
    E2M1_MAX,
    e2m1_value,
    e2m1_decode_table,
    e2m1_encode,
    e8m0_value,
)
from .quant import (
    pow2_exponent,
    pow2_exponents,
    quant_act,
    quant_weight_fp8,
    quant_weight_int4,
    dequant_act,
    dequant_weight_fp8,
    unpack_int4,
    dequant_weight_int4,
    pow2_exponent_e2m1,
    quant_weight_fp4,
    dequant_weight_fp4,
    INT8_MAX,
    quant_int8,
    dequant_int8,
)
from .routing import (
    DEV_ID_RANGE,
    DEV_CAPACITY,
    packed_rows_cap,
    route,
    pack_rows,
)
from .gemm import (grouped_gemm_bf16, grouped_gemm_fp8, grouped_gemm_fp8_fp4, grouped_gemm_int4, grouped_gemm_int8,
                   segments)
from .combine import combine, combine_fp32, f32_to_bf16_bits
from .activation import quant_act_values, silu, swiglu, swiglu_quant
from .metrics import calc_diff, elementwise_ok, elementwise_excess

__all__ = [
    "E4M3_MAX", "e4m3_value", "e4m3_decode_table", "e4m3_encode",
    "bf16_bits_to_f64", "f64_to_bf16_bits", "f64_to_bf16_bits_normal", "fp16_bits_to_f64",
    "pow2_exponent", "pow2_exponents", "quant_act", "quant_weight_fp8",
    "quant_weight_int4", "dequant_act", "dequant_weight_fp8", "unpack_int4",
    "dequant_weight_int4",
    "DEV_ID_RANGE", "DEV_CAPACITY", "packed_rows_cap", "route", "pack_rows",
    "grouped_gemm_bf16", "grouped_gemm_fp8", "grouped_gemm_fp8_fp4", "grouped_gemm_int4", "segments",
    "E2M1_MAX", "e2m1_value", "e2m1_decode_table", "e2m1_encode", "e8m0_value", "pow2_exponent_e2m1",
    "quant_weight_fp4", "dequant_weight_fp4", "combine", "combine_fp32", "f32_to_bf16_bits",
    "calc_diff", "elementwise_ok", "elementwise_excess",
    "silu", "swiglu", "quant_act_values", "swiglu_quant",
    "INT8_MAX", "quant_int8", "dequant_int8", "grouped_gemm_int8",
]
