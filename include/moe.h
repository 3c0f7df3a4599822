/*
 * moe.h -- C ABI of libmoe.so, the MoE grouped-GEMM hot path on gfx950 (MI355X).
 *
 * Data flow of one MoE expert layer (rainlin, "GEMM 执行方式", sec. 4.6 flow:
 * scatter -> grouped GEMM -> gather):
 *
 *   moe_quant_act          bf16 tokens -> FP8 E4M3 codes + 1x128 pow2 scales
 *   moe_route_pack         topk_ids -> per-expert segments; copies token rows
 *   moe_route_pack_quant   (the two steps above in one call) quantises bf16 rows into the segments
 *   moe_grouped_gemm_fp8   packed rows x expert weights (128x128 pow2 scales) -> bf16
 *   moe_grouped_gemm_int4  (weight-only variant) bf16 rows x 4-bit weights -> bf16
 *   moe_grouped_gemm_bf16  (BF16 variant) bf16 rows x bf16 expert weights -> bf16
 *   moe_grouped_gemm_fp8_fp4 (FP4 variant) FP8 rows x MXFP4 (E2M1 + E8M0) weights -> bf16
 *   moe_grouped_gemm_int8  (INT8 variant) int8 rows x int8 weights, (1, 1, 128) fp32 scales -> bf16
 *   moe_swiglu_quant       (between up- and down-projection) silu(gate) * up -> FP8 + 1x128 scales
 *   moe_grouped_gemm_fp8_swiglu (up-projection with the step above in its epilogue) -> FP8 + 1x128 scales
 *   moe_unpermute_combine  topk_weights-weighted sum back to token order
 *
 * plus weight-preparation calls (moe_quant_weight_fp8 / _int4 / _fp4 / _int8,
 * moe_pack_weight_fp8 / _int4 / _fp4 / _bf16) that turn bf16 expert weights
 * into the formats the GEMMs read, and moe_quant_act_int8 (the INT8 variant's
 * activation codes).
 *
 * Conventions for every call:
 *   - All array arguments are DEVICE pointers owned by the caller.  The library
 *     keeps no pointer after the call returns and allocates no device memory;
 *     scratch memory, when needed, is passed in as `workspace`.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued asynchronously; no call synchronises the host.  Buffers must stay
 *     alive until the stream work has finished.
 *   - Arguments are validated on the host before anything is launched.  A
 *     failure returns a nonzero moe_status, launches nothing, and leaves a
 *     human-readable reason in moe_last_error() (thread-local).
 *   - Conditions only the device can see (an expert id >= E, a masked-layout
 *     expert receiving more than max_m rows) are ORed as MOE_DEV_* bits into
 *     *dev_status; the caller zeroes it beforehand and reads it after a sync.
 *   - Row-major layouts everywhere; "bf16" and "fp16" are uint16 bit patterns.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics; the only atomics are order-free integer
 *     counts in LDS).
 *   - Calls on different streams may run concurrently; calls are thread-safe.
 */
#ifndef MOE_H
#define MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;

enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                         */
  MOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent             */
  MOE_ERR_UNSUPPORTED = 3, /* valid in principle, not supported (e.g. K % 128)   */
  MOE_ERR_ALIGN = 4,       /* a pointer or row stride is not aligned as required */
  MOE_ERR_HIP = 5,         /* the HIP runtime reported an error at launch        */
  MOE_ERR_WORKSPACE = 6    /* workspace missing or smaller than required         */
};

/* bits ORed into *dev_status by moe_route_pack */
enum {
  MOE_DEV_ID_RANGE = 1 << 0, /* some topk id was >= E; that route was skipped      */
  MOE_DEV_CAPACITY = 1 << 1  /* masked layout: an expert got more than max_m rows;  */
                             /* the surplus routes were dropped (output_index -1) */
};

enum { MOE_LAYOUT_CONTIGUOUS = 0, MOE_LAYOUT_MASKED = 1 };

/* Flag ORed into the layout argument of moe_grouped_gemm_fp8 (and _int4,
 * _fp8_fp4, _bf16, _int8): the weights are in the fragment-packed order
 * written by moe_pack_weight_fp8 (moe_pack_weight_int4, _fp4, _bf16; the INT8
 * codes use moe_pack_weight_fp8's order) instead of row-major [E, N, K]
 * ([E, N, K/2]). */
enum { MOE_WEIGHTS_PACKED = 0x10 };

enum { MOE_MAX_EXPERTS = 1024, MOE_MAX_TOPK = 64 };

/* Version of this ABI (bumped on any incompatible change). */
int moe_abi_version(void);

/* Static description of a status code. */
const char* moe_status_str(moe_status s);

/* Reason for the most recent failure on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Upper bound on the packed rows of the contiguous layout, computable before
 * routing: every route takes a row and each non-empty expert pads at most
 * align-1 rows (rainlin, "GEMM 执行方式", sec. 4.6: segment length is the count
 * rounded up to the alignment; empty experts take no rows).
 *   = round_up(T*k + min(E, T*k)*(align-1), align).   Returns -1 on bad input. */
int64_t moe_packed_rows_cap(int T, int k, int E, int align);

/* Workspace bytes moe_route_pack needs for (T, k, E); 0 when T*k is small
 * enough for the single-launch path.  Returns -1 on bad input. */
int64_t moe_route_pack_workspace_bytes(int T, int k, int E);

/* ------------------------------------------------------------------------- */
/* moe_quant_act: 1x128 FP8 quantisation of activations.
 * (nxmr.cn DeepGEMM FP8 article, "补偿机制一": every scale factor is an exact
 *  power of two and the quantiser rounds amax/448 up to one; E4M3 range +-448.)
 *   x  [rows, K] bf16.  q [rows, K] E4M3FN codes.  sf [rows, K/128] fp32.
 *   For each row and each 128-wide block along K:
 *     e  = smallest integer with amax <= 448 * 2^e (amax = max |x| of the block),
 *          clamped to [-126, 127]; e = 0 when amax == 0;
 *     sf = 2^e;  q = round-to-nearest-even E4M3 of x * 2^-e (subnormals kept,
 *          sign kept for values that round to zero).
 *   Requires K % 128 == 0, x and q 16-byte aligned, sf 4-byte aligned.
 *   rows == 0 is a no-op. */
moe_status moe_quant_act(const uint16_t* x, int64_t rows, int K,
                         uint8_t* q, float* sf, void* stream);

/* moe_quant_weight_fp8: 128x128 FP8 quantisation of expert weights (same rule
 * per 128x128 block; the article's recipe (gran_m, gran_n, gran_k) with
 * gran_n = gran_k = 128).
 *   w [E, N, K] bf16 -> q [E, N, K] E4M3FN codes, sfw [E, N/128, K/128] fp32.
 *   Requires N % 128 == 0, K % 128 == 0, w and q 16-byte aligned. */
moe_status moe_quant_weight_fp8(const uint16_t* w, int E, int N, int K,
                                uint8_t* q, float* sfw, void* stream);

/* moe_pack_weight_fp8: reorder row-major E4M3 weight codes [E, N, K] into the
 * fragment-packed order the FP8 grouped GEMM reads fastest (a weight layout
 * prepared once, offline, like the prepacked weights of ONNX Runtime
 * "MatMulNBits -- CUDA Operator Documentation" (the weight_prepacked
 * attribute of its fpA_intB path) and the transform-once weight scale
 * layouts of the nxmr.cn DeepGEMM article, "补偿机制三").  Nothing is
 * quantised or rounded: the output is a permutation of the input bytes.
 *   For expert e, K block kb (128 K values), 16-column block cb, half h
 *   (the 64 K values 128kb + 64h ...), lane L = c16 + 16*g (c16 in [0,16),
 *   g in [0,4)) and byte j in [0,16):
 *     packed[e*N*K + ((kb*(N/16) + cb)*2 + h)*1024 + L*16 + j]
 *       = q[e][16*cb + c16][128*kb + 64*h + 16*g + j]
 *   i.e. each 16 x 128 block is 2 KB contiguous, K blocks outermost, so the
 *   columns of one K block are adjacent.  q and packed are [E*N*K] bytes,
 *   16-byte aligned, and must not overlap.  Requires N % 128 == 0, K % 128 == 0.
 *   The scales (sfw) are unchanged. */
moe_status moe_pack_weight_fp8(const uint8_t* q, int E, int N, int K, uint8_t* packed, void* stream);

/* moe_pack_weight_int4: the same idea for 4-bit weights (MatMulNBits codes and
 * scales in, fragment order out; ONNX Runtime "MatMulNBits -- CUDA Operator
 * Documentation" describes prepacked weights for its fpA_intB path).  Nothing
 * is quantised or rounded: weights and scales are only permuted.
 *   Weights, per expert e, K group g (128 weights), 16-column block cb, lane
 *   L = c16 + 16*h (c16, h as above), dword d in [0,4), nibble position p in
 *   [0,8) (bits 4p..4p+3 of the little-endian dword):
 *     weight (n = 16*cb + c16, k = 128*g + 8*(4*d + h) + sigma(p)),
 *     sigma = (0 2 4 6 1 3 5 7), is stored at byte
 *     e*N*K/2 + (g*(N/16) + cb)*1024 + 16*L + 4*d + p/2, low nibble if p is even.
 *   So each dword holds 8 consecutive k of one column, k + 2i and k + 2i + 1
 *   at nibbles i and i + 4.
 *   Scales: s16_packed[e*N*K/128 + ((g*(N/64) + n/64)*16 + n%16)*4 + (n%64)/16]
 *     = s16[e][n][g].
 *   q4/q4_packed are [E*N*K/2] bytes, s16/s16_packed [E*N*K/128] fp16; all
 *   16-byte aligned, inputs and outputs not overlapping.
 *   Requires N % 128 == 0, K % 128 == 0. */
moe_status moe_pack_weight_int4(const uint8_t* q4, const uint16_t* s16, int E, int N, int K, uint8_t* q4_packed,
                                uint16_t* s16_packed, void* stream);

/* moe_quant_weight_int4: group-128 4-bit weight quantisation in the
 * MatMulNBits layout (ONNX Runtime "MatMulNBits -- CUDA Operator
 * Documentation", sec. 2 "Weight Format": row n holds K/2 bytes, two 4-bit
 * weights per byte, one scale per 128 along K, value = (q - 8) * scale).
 * The pages leave the offline scale rule open; this call uses, per (n, group):
 *   s = fp16(fp32(amax) / 7)  (s = 1 when amax == 0; the smallest fp16
 *       subnormal if that underflows to 0; at most 65504),
 *   q = clip(rne(w / s) + 8, 0, 15) with the division in fp32.
 *   w [E, N, K] bf16 -> q4 [E, N, K/2] (low nibble = even k),
 *   s16 [E, N, K/128] fp16.  Requires K % 128 == 0, w 16-byte aligned,
 *   q4 and s16 4-byte aligned. */
moe_status moe_quant_weight_int4(const uint16_t* w, int E, int N, int K,
                                 uint8_t* q4, uint16_t* s16, void* stream);

/* ------------------------------------------------------------------------- */
/* moe_route_pack: routing bookkeeping and packing ("scatter").
 * (rainlin, "GEMM 执行方式", sec. 4.2-4.3 and 4.6; AsymGEMM README, "Token
 *  Layout Protocols"; CuTeDSL bei Perplexity, MoE dispatch: count per expert,
 *  a unique index within the expert, copy into padded buffers.)
 *
 *   topk_ids [T, k] int32.  Route i = t*k + r with 0 <= id < E is valid; ids < 0
 *   are skipped silently, ids >= E are skipped and flag MOE_DEV_ID_RANGE.
 *   Rows within an expert follow route order i (deterministic, bit-exact).
 *
 *   layout MOE_LAYOUT_CONTIGUOUS, align_or_max_m = align (>= 1, e.g. 128):
 *     segment e starts at sum_{e'<e} round_up(count_e', align); empty experts
 *     take no rows.  rows_cap >= moe_packed_rows_cap(T, k, E, align).
 *   layout MOE_LAYOUT_MASKED, align_or_max_m = max_m (>= 1):
 *     segment e starts at e*max_m; an expert's routes beyond the first max_m are
 *     dropped (output_index -1, MOE_DEV_CAPACITY).  rows_cap >= E*max_m.
 *
 *   Outputs:
 *     counts[E]        rows placed in each segment (masked: at most max_m)
 *     seg_offsets[E+1] segment starts; [E] = packed total (masked: E*max_m)
 *     m_indices[rows_cap] expert of each packed row (padding rows included);
 *                      -1 past the packed total
 *     output_index[T,k] packed row of each route, -1 if none
 *     packed  [rows_cap, payload_row_bytes]:   packed[output_index[t,r]] = payload[t]
 *     packed2 [rows_cap, payload2_row_bytes]:  same for a second per-token payload
 *                      (e.g. the FP8 scale rows); pass NULL/0 if unused.
 *   Padding rows of packed/packed2 are never written.
 *   Row byte counts must be multiples of 4; payload/packed must be 16-byte
 *   aligned (payload2/packed2: 4-byte).  workspace: at least
 *   moe_route_pack_workspace_bytes(T, k, E) bytes (may be NULL when that is 0).
 *   Calls that overlap on one stream must not share a workspace. */
moe_status moe_route_pack(const int32_t* topk_ids, int T, int k, int E,
                          int layout, int align_or_max_m,
                          const void* payload, int64_t payload_row_bytes,
                          const void* payload2, int64_t payload2_row_bytes,
                          void* packed, void* packed2, int64_t rows_cap,
                          int32_t* counts, int32_t* seg_offsets,
                          int32_t* m_indices, int32_t* output_index,
                          int32_t* dev_status,
                          void* workspace, int64_t workspace_bytes,
                          void* stream);

/* moe_route_pack_quant: moe_quant_act and moe_route_pack in one call -- the
 * bf16 token rows are quantised (1x128 blocks, power-of-two scales, E4M3
 * codes: exactly the rule of moe_quant_act, nxmr.cn DeepGEMM article,
 * "补偿机制一") on the way into the packed layout, so the token-order codes
 * are never written to HBM and read back (rainlin, "GEMM 执行方式", sec. 4.6
 * flow: scatter -> grouped GEMM -> gather, with the quantisation folded into
 * the scatter).
 *   x [T, K] bf16 (16-byte aligned, K % 128 == 0, K <= 32768); packed_q [rows_cap, K]
 *   E4M3 codes (16-byte aligned) and packed_sf [rows_cap, K/128] fp32 scales
 *   (4-byte aligned) receive what moe_route_pack would copy from
 *   moe_quant_act's q and sf (payload = q, payload2 = sf), bit for bit; every
 *   other argument, output, error and the workspace as for moe_route_pack.
 *   Each token's row is quantised once however many experts it is routed to. */
moe_status moe_route_pack_quant(const int32_t* topk_ids, int T, int k, int E,
                                int layout, int align_or_max_m,
                                const uint16_t* x, int K,
                                uint8_t* packed_q, float* packed_sf, int64_t rows_cap,
                                int32_t* counts, int32_t* seg_offsets,
                                int32_t* m_indices, int32_t* output_index,
                                int32_t* dev_status,
                                void* workspace, int64_t workspace_bytes,
                                void* stream);

/* moe_route_pack_noalloc: moe_route_pack for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, results and errors, minus the
 * workspace.  The scratch the large-T*k path needs lives in one fixed device
 * array inside the library, moe_route_pack_noalloc_max_bytes() bytes (4 MiB)
 * per device, held until the process ends; calls whose
 * moe_route_pack_workspace_bytes(T, k, E) exceeds it fail with
 * MOE_ERR_WORKSPACE before anything is launched (4 MiB covers, e.g., 1M
 * routes over 1024 experts or 8M routes over 128).  The call allocates
 * nothing: no hipMalloc, no hipFree, no allocating library routine.  Every
 * call on one device shares that device's array, so calls that overlap in
 * time on one device (different streams, or different host threads) race and
 * must be serialised by the caller; calls on different devices do not
 * interact.  Nothing in the array needs clearing between calls. */
int64_t moe_route_pack_noalloc_max_bytes(void);
moe_status moe_route_pack_noalloc(const int32_t* topk_ids, int T, int k, int E,
                                  int layout, int align_or_max_m,
                                  const void* payload, int64_t payload_row_bytes,
                                  const void* payload2, int64_t payload2_row_bytes,
                                  void* packed, void* packed2, int64_t rows_cap,
                                  int32_t* counts, int32_t* seg_offsets,
                                  int32_t* m_indices, int32_t* output_index,
                                  int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------- */
/* moe_grouped_gemm_fp8: block-scaled FP8 grouped GEMM, "NT" (both operands
 * K-contiguous).  (rainlin, "GEMM 执行方式", sec. 4.1/4.4: Y_e = X_e W_e^T per
 *  expert; AsymGEMM README, "API Reference" (m_grouped_fp8 contiguous/masked,
 *  (data, scale) operands, bf16 output) and "asymScheduler" (each workgroup
 *  owns expert tiles, no atomics); nxmr.cn DeepGEMM article: FP32 accumulation
 *  with per-block scales.)
 *
 *   For every segment e and row p in [start_e, start_e + counts[e]):
 *     D[p, n] = bf16_rne( sum_kb sa[p,kb] * sw[e, n/128, kb] *
 *                         sum_{k in kb} dec(A[p,k]) * dec(W[e,n,k]) )
 *   accumulated in fp32 (the per-128-K-block scales are applied inside the
 *   matrix instruction, which is exact for powers of two).
 *     A   [rows, K] E4M3FN, SFA [rows, K/128] fp32 powers of two
 *     W   [E, N, K] E4M3FN, SFW [E, N/128, K/128] fp32 powers of two
 *     D   [rows, N] bf16
 *   layout CONTIGUOUS: start_e = seg_offsets[e], rows_cap_or_max_m = rows of A/D.
 *   layout MASKED:     start_e = e*max_m, rows_cap_or_max_m = max_m,
 *                      seg_offsets ignored (may be NULL), rows = E*max_m.
 *   layout | MOE_WEIGHTS_PACKED: W holds the codes in the order written by
 *                      moe_pack_weight_fp8 (same values, faster to stream).
 *   counts[e] is clipped to the segment capacity on the device.
 *   expected_m: tiling hint, the mean rows per active expert (0 = choose from
 *   the layout).  Rows of D outside the segments are never written.
 *   Requires K % 128 == 0, N % 128 == 0, 1 <= E <= 1024, A/W/D 16-byte aligned. */
moe_status moe_grouped_gemm_fp8(int layout,
                                const uint8_t* A, const float* SFA,
                                const uint8_t* W, const float* SFW,
                                uint16_t* D,
                                const int32_t* counts, const int32_t* seg_offsets,
                                int E, int64_t rows_cap_or_max_m, int N, int K,
                                int expected_m, void* stream);

/* moe_grouped_gemm_int4: 4-bit weight-only grouped GEMM (ONNX Runtime
 * "MatMulNBits -- CUDA Operator Documentation", sec. 2: (q - 8) * scale with
 * group 128 along K).
 *     D[p, n] = bf16_rne( sum_g s[e,n,g] * sum_{k in g} A[p,k] * (q[e,n,k] - 8) )
 *   accumulated in fp32.
 *     A   [rows, K] bf16,  W4 [E, N, K/2] (low nibble = even k),
 *     S16 [E, N, K/128] fp16,  D [rows, N] bf16.
 *   Layout, counts, seg_offsets, expected_m and alignment as for
 *   moe_grouped_gemm_fp8 (S16 2-byte aligned); layout | MOE_WEIGHTS_PACKED: W4
 *   and S16 in the orders written by moe_pack_weight_int4, S16 8-byte aligned. */
moe_status moe_grouped_gemm_int4(int layout,
                                 const uint16_t* A, const uint8_t* W4,
                                 const uint16_t* S16, uint16_t* D,
                                 const int32_t* counts, const int32_t* seg_offsets,
                                 int E, int64_t rows_cap_or_max_m, int N, int K,
                                 int expected_m, void* stream);

/* moe_pack_weight_bf16: reorder bf16 expert weights [E, N, K] into the
 * fragment-packed order the BF16 grouped GEMM streams fastest: the weight
 * bytes, viewed as [E, N, 2K], in moe_pack_weight_fp8's order with 2K in place
 * of K (each 16-column x 128-byte block, i.e. 64 bf16 values of 16 columns,
 * is 2 KB contiguous, K blocks outermost).  A permutation of the 16-bit
 * values; nothing is rounded.  Requires N % 128 == 0, K % 128 == 0, both
 * buffers 16-byte aligned and not overlapping. */
moe_status moe_pack_weight_bf16(const uint16_t* w, int E, int N, int K, uint16_t* packed, void* stream);

/* moe_grouped_gemm_bf16: BF16 grouped GEMM, "NT" (both operands
 * K-contiguous).  (AsymGEMM README, "API Reference": BF16 m_grouped
 * contiguous and masked grouped GEMMs with bf16 output; rainlin, "GEMM
 * 执行方式", sec. 4.6: the BF16 contiguous grouped GEMM on the packed segments.)
 *     D[p, n] = bf16_rne( sum_k A[p,k] * W[e,n,k] ), accumulated in fp32.
 *     A [rows, K] bf16, W [E, N, K] bf16, D [rows, N] bf16.
 *   Layout, counts, seg_offsets, expected_m, the rows of D that are written,
 *   alignment and size limits as for moe_grouped_gemm_fp8; layout |
 *   MOE_WEIGHTS_PACKED: W in the order written by moe_pack_weight_bf16. */
moe_status moe_grouped_gemm_bf16(int layout,
                                 const uint16_t* A, const uint16_t* W, uint16_t* D,
                                 const int32_t* counts, const int32_t* seg_offsets,
                                 int E, int64_t rows_cap_or_max_m, int N, int K,
                                 int expected_m, void* stream);

/* moe_quant_weight_fp4: MXFP4 quantisation of expert weights for
 * moe_grouped_gemm_fp8_fp4 (AsymGEMM README, "API Reference": FP4 weights as
 * packed 4-bit data plus scales; CuTeDSL bei Perplexity: the MXFP4 block
 * scaling).  Per output column n and block of 32 consecutive k: amax; e = the
 * smallest integer with amax <= 6 * 2^e, clamped to [-127, 127], 0 when
 * amax == 0 (the pages give no offline rule: the FP8 rule with the E2M1
 * maximum 6); sw = e + 127 (an E8M0 byte); codes = E2M1 round-to-nearest-even
 * of w * 2^-e (sign kept for values that round to zero).
 *   w [E, N, K] bf16 -> w4 [E, N, K/2] (two codes per byte, the even k in the
 *   low nibble), sw [E, N, K/32] E8M0 bytes.
 *   Requires K % 128 == 0, w and w4 16-byte aligned. */
moe_status moe_quant_weight_fp4(const uint16_t* w, int E, int N, int K,
                                uint8_t* w4, uint8_t* sw, void* stream);

/* moe_pack_weight_fp4: reorder MXFP4 weights (moe_quant_weight_fp4's codes and
 * E8M0 scales) into the fragment-packed orders the FP8 x FP4 grouped GEMM
 * streams fastest (a layout prepared once, offline, as moe_pack_weight_fp8).
 * Nothing is quantised or rounded: codes and scales are only permuted.
 *   Codes: for expert e, step ks (128 K values), 16-column block cb and lane
 *   L = c16 + 16*g (c16 in [0,16), g in [0,4)), the 16 bytes of column
 *   16*cb + c16, K = 128*ks + 32*g .. +31 (row-major bytes
 *   w4[e][n][64*ks + 16*g .. +15]) are stored at
 *     w4_packed[e*N*K/2 + ((ks*(N/16) + cb)*64 + L)*16].
 *   Scales: for expert e, step ks, 64-column group n64 and lane L, byte j of
 *   the dword at sw_packed[e*N*K/32 + ((ks*(N/64) + n64)*64 + L)*4] is the
 *   scale of column 64*n64 + 16*j + c16, block 4*ks + g:
 *     sw_packed[... + j] = sw[e][64*n64 + 16*j + c16][4*ks + g],   j in [0,4).
 *   Requires N % 128 == 0 and K % 128 == 0; codes 16-byte aligned, scales
 *   4-byte aligned; outputs must not overlap any buffer. */
moe_status moe_pack_weight_fp4(const uint8_t* w4, const uint8_t* sw, int E, int N, int K,
                               uint8_t* w4_packed, uint8_t* sw_packed, void* stream);

/* moe_grouped_gemm_fp8_fp4: FP8 activations x MXFP4 weights grouped GEMM
 * (AsymGEMM README, "API Reference": FP4 m_grouped contiguous and masked
 * grouped GEMMs; nxmr.cn DeepGEMM article, "精度与吞吐的平衡点": a product with
 * one FP4 operand is held to calc_diff < 0.01).
 *   For every segment e and row p in [start_e, start_e + counts[e]):
 *     D[p, n] = bf16_rne( sum_k (dec(A[p,k]) * SFA[p, k/128]) *
 *                         (e2m1(W4[e,n,k]) * 2^(SW[e,n,k/32] - 127)) )
 *   accumulated in fp32, the power-of-two scales applied inside the matrix
 *   instruction (exact).
 *     A [rows, K] E4M3FN, SFA [rows, K/128] fp32 powers of two (moe_quant_act);
 *     W4 [E, N, K/2] and SW [E, N, K/32] as written by moe_quant_weight_fp4;
 *     D [rows, N] bf16.
 *   Layout, counts, seg_offsets, expected_m, the rows of D that are written,
 *   alignment (SFA and SW 4-byte aligned) and size limits as for
 *   moe_grouped_gemm_fp8.  layout | MOE_WEIGHTS_PACKED: W4 and SW in the
 *   orders written by moe_pack_weight_fp4. */
moe_status moe_grouped_gemm_fp8_fp4(int layout,
                                    const uint8_t* A, const float* SFA,
                                    const uint8_t* W4, const uint8_t* SW,
                                    uint16_t* D,
                                    const int32_t* counts, const int32_t* seg_offsets,
                                    int E, int64_t rows_cap_or_max_m, int N, int K,
                                    int expected_m, void* stream);

/* ------------------------------------------------------------------------- */
/* INT8 (1, 1, 128) variant (AsymGEMM README, "API Reference", INT8 asymmetric
 * GEMM: int8 data paired with fp32 scales of fixed granularity (1, 1, 128):
 * one scale per token row and 128 K for the activations, one per output
 * channel and 128 K for the weights; contiguous and masked grouped layouts,
 * bf16 output).  The page fixes no rule for choosing a scale; these calls use
 * the symmetric one: s = amax / 127 over the 128-element block (fp32,
 * correctly rounded division; s = 1 for an all-zero block) and codes
 * rne(x / s) (the same division) clamped to [-127, 127].
 *
 * moe_quant_act_int8: x [rows, K] bf16 -> q [rows, K] int8 and
 *   s [rows, K/128] fp32.  Requires K % 128 == 0; x and q 16-byte aligned, s
 *   4-byte aligned; rows == 0 is a no-op.  Outputs must not overlap x. */
moe_status moe_quant_act_int8(const uint16_t* x, int64_t rows, int K, int8_t* q, float* s, void* stream);

/* moe_quant_weight_int8: expert weights w [E, N, K] bf16 -> q [E, N, K] int8
 *   (row n of expert e quantised as one activation row) and the per-channel
 *   scales in the K-block-major order the grouped GEMM reads:
 *   sw[(e * K/128 + kb) * N + n] is the scale of q[e, n, 128kb .. 128kb+127]
 *   (the page's [E, N, K/128] scales transposed in their last two dimensions).
 *   Requires N % 128 == 0 and K % 128 == 0; w and q 16-byte aligned, sw
 *   4-byte aligned; E == 0 is a no-op.  q may be passed to
 *   moe_pack_weight_fp8 (a byte permutation) for the packed weight order. */
moe_status moe_quant_weight_int8(const uint16_t* w, int E, int N, int K, int8_t* q, float* sw, void* stream);

/* moe_grouped_gemm_int8: int8 activations x int8 weights grouped GEMM.
 *   For every segment e and row p in [start_e, start_e + counts[e]):
 *     D[p, n] = bf16_rne( sum_kb SA[p, kb] * SW[e, kb, n] *
 *                         sum_{k in block kb} A[p, k] * W[e, n, k] )
 *   each block's integer sum exact, the scaled sums accumulated in fp32.
 *     A [rows, K] int8, SA [rows, K/128] fp32 (moe_quant_act_int8);
 *     W [E, N, K] int8, SW [E, K/128, N] fp32 (moe_quant_weight_int8);
 *     D [rows, N] bf16.
 *   Layout, counts, seg_offsets, expected_m, the rows of D that are written,
 *   and size limits as for moe_grouped_gemm_fp8; SA 4-byte aligned, SW
 *   16-byte aligned.  layout | MOE_WEIGHTS_PACKED: W in the fragment order of
 *   moe_pack_weight_fp8 (SW unchanged). */
moe_status moe_grouped_gemm_int8(int layout,
                                 const int8_t* A, const float* SA,
                                 const int8_t* W, const float* SW,
                                 uint16_t* D,
                                 const int32_t* counts, const int32_t* seg_offsets,
                                 int E, int64_t rows_cap_or_max_m, int N, int K,
                                 int expected_m, void* stream);

/* ------------------------------------------------------------------------- */
/* moe_swiglu_quant: SwiGLU between the up- and down-projection, requantised
 * for the down-projection's FP8 GEMM.  (The pages' fused gate+up expert weight
 * -- a DeepSeek-V3-shaped up-projection has 2 x 2048 output columns -- and
 * the activation kernels CuTeDSL bei Perplexity lists among the MoE kernels;
 * the requantisation is the 1x128 rule of moe_quant_act, nxmr.cn DeepGEMM FP8
 * article, "补偿机制一".)
 *   gate_up [rows, 2I] bf16: the up-projection's output, gate in columns
 *   0..I-1 and up in columns I..2I-1.  For every row p of every segment (the
 *   same segments and clipping as moe_grouped_gemm_fp8: contiguous
 *   rows_cap_or_max_m = rows and start_e = seg_offsets[e]; masked
 *   rows_cap_or_max_m = max_m and start_e = e*max_m):
 *     h[p, j] = silu(gate[p, j]) * up[p, j],  silu(x) = x / (1 + exp(-x)),
 *   evaluated in fp32 (t = exp(-g) by the hardware exp2 of -g*log2(e), the
 *   product carried with its rounding error; s = g * rcp(1 + t); h = s * u;
 *   a few fp32 ulps from the exact value), then per
 *   128-column block: sf = 2^e with e the smallest integer with
 *   amax|h| <= 448 * 2^e (clamped to [-126, 127], 0 when amax == 0) and
 *   q = round-to-nearest-even E4M3 of h * 2^-e.  h is never rounded to bf16.
 *     q [rows, I] E4M3FN codes, sf [rows, I/128] fp32 powers of two.
 *   Rows outside the segments are neither read nor written.
 *   Requires I % 128 == 0, gate_up and q 16-byte aligned, sf 4-byte aligned. */
moe_status moe_swiglu_quant(int layout, const uint16_t* gate_up, int64_t rows_cap_or_max_m, int I,
                            const int32_t* counts, const int32_t* seg_offsets, int E,
                            uint8_t* q, float* sf, void* stream);

/* moe_grouped_gemm_fp8_swiglu: the up-projection's FP8 grouped GEMM with
 * SwiGLU and the 1x128 requantisation in its epilogue, so the [rows, 2I] bf16
 * gate/up output never goes through HBM (the same sources as
 * moe_grouped_gemm_fp8 and moe_swiglu_quant).
 *   The result is, bit for bit, that of moe_grouped_gemm_fp8 with N = 2I
 *   into a bf16 gate_up followed by moe_swiglu_quant on it: every gate and up
 *   value is the GEMM's fp32 accumulation rounded to bf16 (nearest even),
 *   then h = silu(gate) * up in fp32 and the 1x128 power-of-two quantisation
 *   exactly as moe_swiglu_quant computes them.
 *     A [rows, K] E4M3FN, SFA [rows, K/128] fp32 powers of two (moe_quant_act);
 *     W [E, 2I, K] E4M3FN, SFW [E, 2I/128, K/128] fp32 powers of two: the
 *       gate rows 0..I-1, then the up rows I..2I-1 (the weight of the plain
 *       up-projection; layout | MOE_WEIGHTS_PACKED: in the order written by
 *       moe_pack_weight_fp8 with N = 2I);
 *     Q [rows, I] E4M3FN codes, SQ [rows, I/128] fp32 powers of two.
 *   Layout, counts, seg_offsets and expected_m as for moe_grouped_gemm_fp8;
 *   rows of Q and SQ outside the segments are never written.
 *   Requires I % 128 == 0, K % 512 == 0 (K <= 32768), 1 <= E <= 1024, A, W and
 *   Q 16-byte aligned, SFA 16-byte and SFW, SQ 4-byte aligned; otherwise
 *   MOE_ERR_UNSUPPORTED / MOE_ERR_ALIGN and nothing is launched. */
moe_status moe_grouped_gemm_fp8_swiglu(int layout,
                                       const uint8_t* A, const float* SFA,
                                       const uint8_t* W, const float* SFW,
                                       uint8_t* Q, float* SQ,
                                       const int32_t* counts, const int32_t* seg_offsets,
                                       int E, int64_t rows_cap_or_max_m, int I, int K,
                                       int expected_m, void* stream);

/* ------------------------------------------------------------------------- */
/* moe_unpermute_combine: weighted combine back to token order ("gather").
 * (rainlin, "GEMM 执行方式", sec. 4.4 and 4.6: z_t = sum_r p[t,r] *
 *  y_packed[output_index[t,r]], reading only rows named by output_index;
 *  CuTeDSL bei Perplexity: the combine accumulates in registers.)
 *     Z[t, n] = bf16_rne( fma-chain over r = 0..k-1 of p[t,r] * Y[output_index[t,r], n] )
 *   in fp32, slot order r = 0..k-1; slots with output_index < 0 or >= y_rows
 *   contribute nothing.  Weights are used as given.
 *     Y [y_rows, N] bf16, output_index [T, k] int32, topk_weights [T, k] fp32,
 *     Z [T, N] bf16.  Requires N % 8 == 0, Y and Z 16-byte aligned. */
moe_status moe_unpermute_combine(const uint16_t* Y, int64_t y_rows,
                                 const int32_t* output_index,
                                 const float* topk_weights,
                                 int T, int k, int N,
                                 uint16_t* Z, void* stream);

/* moe_stream_read: a measurement helper, not a step of the method.  Reads the
 * `bytes` bytes at `buf` once with 16-byte nontemporal loads (eight in
 * flight per lane, one 256-lane workgroup per compute unit) and writes an XOR fold
 * of every 32-bit word read to out[0 .. moe_stream_read_words() - 1] (one
 * word per workgroup; the XOR of all of them is the XOR of the buffer), so
 * that the reads cannot be dropped.  Timing it gives the HBM read rate the
 * memory-bound kernels are compared with besides the nominal peak.
 *   Requires bytes % 16 == 0, buf 16-byte and out 4-byte aligned (device
 *   pointers owned by the caller); bytes == 0 writes zeros. */
int moe_stream_read_words(void);
moe_status moe_stream_read(const void* buf, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
