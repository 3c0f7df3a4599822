// api.hip -- the extern "C" boundary of libmoe.so (declared in include/moe.h).
// Every entry point validates its arguments on the host, returns a status
// without launching anything on failure (with a reason in moe_last_error()),
// and otherwise enqueues its kernels on the caller's stream.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/moe.h"
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

static thread_local char g_err[512];

static moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

static moe_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

DeviceInfo device_info() {
  static std::mutex mu;
  static int cached_cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64 && cached_cus[dev] > 0) return DeviceInfo{cached_cus[dev]};
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 64) cached_cus[dev] = cus;
  return DeviceInfo{cus};
}

static bool aligned(const void* p, uintptr_t a) { return (((uintptr_t)p) & (a - 1)) == 0; }

}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return 2; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "bad shape";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_ALIGN: return "misaligned pointer or row";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

int64_t moe_packed_rows_cap(int T, int k, int E, int align) {
  if (T < 0 || k < 1 || E < 1 || align < 1) return -1;
  const int64_t R = (int64_t)T * k;
  const int64_t cap = R + (R < E ? R : E) * (int64_t)(align - 1);
  return (cap + align - 1) / align * align;
}

int64_t moe_route_pack_workspace_bytes(int T, int k, int E) {
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return -1;
  const int64_t R = (int64_t)T * k;
  if (R > 0x7fffffff) return -1;
  return route_workspace_bytes((int)R, E);
}

moe_status moe_quant_act(const uint16_t* x, int64_t rows, int K, uint8_t* q, float* sf, void* stream) {
  g_err[0] = 0;
  if (rows < 0 || K <= 0) return fail(MOE_ERR_SHAPE, "moe_quant_act: rows=%lld K=%d", (long long)rows, K);
  if (K % 128) return fail(MOE_ERR_UNSUPPORTED, "moe_quant_act: K=%d is not a multiple of 128", K);
  if (rows == 0) return MOE_OK;
  if (!x || !q || !sf) return fail(MOE_ERR_NULL, "moe_quant_act: null pointer");
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(sf, 4))
    return fail(MOE_ERR_ALIGN, "moe_quant_act: x and q must be 16-byte aligned, sf 4-byte aligned");
  return hip_status(launch_quant_act(x, rows, K, q, sf, (hipStream_t)stream), "moe_quant_act");
}

moe_status moe_quant_weight_fp8(const uint16_t* w, int E, int N, int K, uint8_t* q, float* sfw, void* stream) {
  g_err[0] = 0;
  if (E < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_SHAPE, "moe_quant_weight_fp8: E=%d N=%d K=%d", E, N, K);
  if (N % 128 || K % 128)
    return fail(MOE_ERR_UNSUPPORTED, "moe_quant_weight_fp8: N=%d and K=%d must be multiples of 128", N, K);
  if (E == 0) return MOE_OK;
  if (!w || !q || !sfw) return fail(MOE_ERR_NULL, "moe_quant_weight_fp8: null pointer");
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(sfw, 4))
    return fail(MOE_ERR_ALIGN, "moe_quant_weight_fp8: w and q must be 16-byte aligned");
  return hip_status(launch_quant_weight_fp8(w, E, N, K, q, sfw, (hipStream_t)stream), "moe_quant_weight_fp8");
}

moe_status moe_pack_weight_fp8(const uint8_t* q, int E, int N, int K, uint8_t* packed, void* stream) {
  g_err[0] = 0;
  if (E < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_SHAPE, "moe_pack_weight_fp8: E=%d N=%d K=%d", E, N, K);
  if (N % 128 || K % 128)
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_weight_fp8: N=%d and K=%d must be multiples of 128", N, K);
  if ((int64_t)N * K > 0xffffffffll) return fail(MOE_ERR_UNSUPPORTED, "moe_pack_weight_fp8: one expert exceeds 4 GiB");
  if (E == 0) return MOE_OK;
  if (!q || !packed) return fail(MOE_ERR_NULL, "moe_pack_weight_fp8: null pointer");
  if (!aligned(q, 16) || !aligned(packed, 16))
    return fail(MOE_ERR_ALIGN, "moe_pack_weight_fp8: q and packed must be 16-byte aligned");
  const uint8_t* qe = q + (int64_t)E * N * K;
  const uint8_t* pe = packed + (int64_t)E * N * K;
  if (q < pe && packed < qe) return fail(MOE_ERR_SHAPE, "moe_pack_weight_fp8: q and packed overlap");
  return hip_status(launch_pack_weight_fp8(q, E, N, K, packed, (hipStream_t)stream), "moe_pack_weight_fp8");
}

moe_status moe_pack_weight_int4(const uint8_t* q4, const uint16_t* s16, int E, int N, int K, uint8_t* q4_packed,
                                uint16_t* s16_packed, void* stream) {
  g_err[0] = 0;
  if (E < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_SHAPE, "moe_pack_weight_int4: E=%d N=%d K=%d", E, N, K);
  if (N % 128 || K % 128)
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_weight_int4: N=%d and K=%d must be multiples of 128", N, K);
  if ((int64_t)N * K / 2 > 0xffffffffll) return fail(MOE_ERR_UNSUPPORTED, "moe_pack_weight_int4: one expert exceeds 4 GiB");
  if (E == 0) return MOE_OK;
  if (!q4 || !s16 || !q4_packed || !s16_packed) return fail(MOE_ERR_NULL, "moe_pack_weight_int4: null pointer");
  if (!aligned(q4, 16) || !aligned(q4_packed, 16) || !aligned(s16, 16) || !aligned(s16_packed, 16))
    return fail(MOE_ERR_ALIGN, "moe_pack_weight_int4: all four buffers must be 16-byte aligned");
  const uint8_t* ranges[4][2] = {{q4, q4 + (int64_t)E * N * (K / 2)},
                                 {(const uint8_t*)s16, (const uint8_t*)(s16 + (int64_t)E * N * (K / 128))},
                                 {q4_packed, q4_packed + (int64_t)E * N * (K / 2)},
                                 {(const uint8_t*)s16_packed, (const uint8_t*)(s16_packed + (int64_t)E * N * (K / 128))}};
  for (int i = 0; i < 2; ++i)
    for (int j = 2; j < 4; ++j)
      if (ranges[i][0] < ranges[j][1] && ranges[j][0] < ranges[i][1])
        return fail(MOE_ERR_SHAPE, "moe_pack_weight_int4: an input overlaps an output");
  if (ranges[2][0] < ranges[3][1] && ranges[3][0] < ranges[2][1])
    return fail(MOE_ERR_SHAPE, "moe_pack_weight_int4: the two outputs overlap");
  return hip_status(launch_pack_weight_int4(q4, s16, E, N, K, q4_packed, s16_packed, (hipStream_t)stream),
                    "moe_pack_weight_int4");
}

moe_status moe_quant_weight_int4(const uint16_t* w, int E, int N, int K, uint8_t* q4, uint16_t* s16, void* stream) {
  g_err[0] = 0;
  if (E < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_SHAPE, "moe_quant_weight_int4: E=%d N=%d K=%d", E, N, K);
  if (K % 128) return fail(MOE_ERR_UNSUPPORTED, "moe_quant_weight_int4: K=%d is not a multiple of 128", K);
  if (E == 0) return MOE_OK;
  if (!w || !q4 || !s16) return fail(MOE_ERR_NULL, "moe_quant_weight_int4: null pointer");
  if (!aligned(w, 16) || !aligned(q4, 4) || !aligned(s16, 2))
    return fail(MOE_ERR_ALIGN, "moe_quant_weight_int4: w must be 16-byte aligned, q4 4-byte aligned");
  return hip_status(launch_quant_weight_int4(w, E, N, K, q4, s16, (hipStream_t)stream), "moe_quant_weight_int4");
}

}  // extern "C"

// Validation shared by moe_route_pack and moe_route_pack_noalloc; fills `a` (workspace left unset).
static moe_status check_route(const char* fn, const int32_t* topk_ids, int T, int k, int E, int layout,
                              int align_or_max_m, const void* payload, int64_t payload_row_bytes,
                              const void* payload2, int64_t payload2_row_bytes, void* packed, void* packed2,
                              int64_t rows_cap, int32_t* counts, int32_t* seg_offsets, int32_t* m_indices,
                              int32_t* output_index, int32_t* dev_status, RouteArgs& a) {
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_SHAPE, "%s: T=%d k=%d E=%d (need T>=0, 1<=k<=%d, 1<=E<=%d)", fn, T, k, E, MOE_MAX_TOPK,
                MOE_MAX_EXPERTS);
  if ((int64_t)T * k > 0x7fffffff) return fail(MOE_ERR_SHAPE, "%s: T*k too large", fn);
  if (layout != MOE_LAYOUT_CONTIGUOUS && layout != MOE_LAYOUT_MASKED)
    return fail(MOE_ERR_SHAPE, "%s: unknown layout %d", fn, layout);
  if (align_or_max_m < 1) return fail(MOE_ERR_SHAPE, "%s: align/max_m=%d must be >= 1", fn, align_or_max_m);
  if (payload_row_bytes <= 0 || payload_row_bytes % 4)
    return fail(MOE_ERR_ALIGN, "%s: payload_row_bytes=%lld must be a positive multiple of 4", fn,
                (long long)payload_row_bytes);
  if (payload2 && (payload2_row_bytes <= 0 || payload2_row_bytes % 4))
    return fail(MOE_ERR_ALIGN, "%s: payload2_row_bytes=%lld must be a positive multiple of 4", fn,
                (long long)payload2_row_bytes);
  const bool any_routes = T > 0;
  if (any_routes && (!topk_ids || !payload || !output_index))
    return fail(MOE_ERR_NULL, "%s: topk_ids, payload and output_index are required when T > 0", fn);
  if (!counts || !seg_offsets || !dev_status) return fail(MOE_ERR_NULL, "%s: null pointer", fn);
  if (rows_cap > 0 && (!packed || !m_indices))
    return fail(MOE_ERR_NULL, "%s: packed and m_indices are required when rows_cap > 0", fn);
  if (payload2 && !packed2) return fail(MOE_ERR_NULL, "%s: packed2 is null but payload2 is not", fn);
  const int64_t need = (layout == MOE_LAYOUT_CONTIGUOUS) ? moe_packed_rows_cap(T, k, E, align_or_max_m)
                                                          : (int64_t)E * align_or_max_m;
  if (rows_cap < need || rows_cap > 0x7fffffff)
    return fail(MOE_ERR_SHAPE, "%s: rows_cap=%lld, need at least %lld (and < 2^31)", fn, (long long)rows_cap,
                (long long)need);
  if (!aligned(payload, 16) || !aligned(packed, 16) || (payload2 && (!aligned(payload2, 4) || !aligned(packed2, 4))))
    return fail(MOE_ERR_ALIGN, "%s: payload/packed must be 16-byte aligned, payload2/packed2 4-byte", fn);
  if (!aligned(topk_ids, 4) || !aligned(counts, 4) || !aligned(seg_offsets, 4) || !aligned(m_indices, 4) ||
      !aligned(output_index, 4) || !aligned(dev_status, 4))
    return fail(MOE_ERR_ALIGN, "%s: int32 arrays must be 4-byte aligned", fn);
  a.ids = topk_ids;
  a.T = T;
  a.k = k;
  a.E = E;
  a.R = T * k;
  a.masked = layout == MOE_LAYOUT_MASKED;
  a.align = a.masked ? 1 : align_or_max_m;
  a.max_m = a.masked ? align_or_max_m : 0;
  a.payload = (const uint8_t*)payload;
  a.row_bytes = payload_row_bytes;
  a.payload2 = (const uint8_t*)payload2;
  a.row_bytes2 = payload2 ? payload2_row_bytes : 0;
  a.packed = (uint8_t*)packed;
  a.packed2 = (uint8_t*)packed2;
  a.rows_cap = rows_cap;
  a.counts = counts;
  a.seg_offsets = seg_offsets;
  a.m_indices = m_indices;
  a.output_index = output_index;
  a.dev_status = dev_status;
  a.ws = nullptr;
  a.nchunks = 0;
  a.xq = nullptr;  // copy the payload rows (moe_route_pack_quant sets the quantising source)
  a.K = 0;
  return MOE_OK;
}

extern "C" {

moe_status moe_route_pack(const int32_t* topk_ids, int T, int k, int E, int layout, int align_or_max_m,
                          const void* payload, int64_t payload_row_bytes, const void* payload2,
                          int64_t payload2_row_bytes, void* packed, void* packed2, int64_t rows_cap, int32_t* counts,
                          int32_t* seg_offsets, int32_t* m_indices, int32_t* output_index, int32_t* dev_status,
                          void* workspace, int64_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  RouteArgs a{};
  moe_status st = check_route("moe_route_pack", topk_ids, T, k, E, layout, align_or_max_m, payload,
                              payload_row_bytes, payload2, payload2_row_bytes, packed, packed2, rows_cap, counts,
                              seg_offsets, m_indices, output_index, dev_status, a);
  if (st) return st;
  const int64_t ws_need = route_workspace_bytes(a.R, E);
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need || !aligned(workspace, 4)))
    return fail(MOE_ERR_WORKSPACE, "moe_route_pack: needs %lld workspace bytes, got %lld", (long long)ws_need,
                (long long)workspace_bytes);
  a.ws = (int32_t*)workspace;
  return hip_status(launch_route_pack(a, (hipStream_t)stream), "moe_route_pack");
}

moe_status moe_route_pack_quant(const int32_t* topk_ids, int T, int k, int E, int layout, int align_or_max_m,
                                const uint16_t* x, int K, uint8_t* packed_q, float* packed_sf, int64_t rows_cap,
                                int32_t* counts, int32_t* seg_offsets, int32_t* m_indices, int32_t* output_index,
                                int32_t* dev_status, void* workspace, int64_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (K <= 0 || K % 128 || K / 128 > kMaxKBlocks)
    return fail(MOE_ERR_UNSUPPORTED, "moe_route_pack_quant: K=%d must be a positive multiple of 128 up to %d", K,
                kMaxKBlocks * 128);
  if (rows_cap > 0 && !packed_sf) return fail(MOE_ERR_NULL, "moe_route_pack_quant: packed_sf is null");
  if (!aligned(packed_sf, 4)) return fail(MOE_ERR_ALIGN, "moe_route_pack_quant: packed_sf must be 4-byte aligned");
  RouteArgs a{};
  moe_status st = check_route("moe_route_pack_quant", topk_ids, T, k, E, layout, align_or_max_m, x, 2 * (int64_t)K,
                              nullptr, 0, packed_q, nullptr, rows_cap, counts, seg_offsets, m_indices, output_index,
                              dev_status, a);
  if (st) return st;
  const int64_t ws_need = route_workspace_bytes(a.R, E);
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need || !aligned(workspace, 4)))
    return fail(MOE_ERR_WORKSPACE, "moe_route_pack_quant: needs %lld workspace bytes, got %lld", (long long)ws_need,
                (long long)workspace_bytes);
  a.ws = (int32_t*)workspace;
  a.xq = x;
  a.K = K;
  a.packed2 = (uint8_t*)packed_sf;
  return hip_status(launch_route_pack(a, (hipStream_t)stream), "moe_route_pack_quant");
}

int64_t moe_route_pack_noalloc_max_bytes(void) { return route_scratch_bytes(); }

moe_status moe_route_pack_noalloc(const int32_t* topk_ids, int T, int k, int E, int layout, int align_or_max_m,
                                  const void* payload, int64_t payload_row_bytes, const void* payload2,
                                  int64_t payload2_row_bytes, void* packed, void* packed2, int64_t rows_cap,
                                  int32_t* counts, int32_t* seg_offsets, int32_t* m_indices, int32_t* output_index,
                                  int32_t* dev_status, void* stream) {
  g_err[0] = 0;
  RouteArgs a{};
  moe_status st = check_route("moe_route_pack_noalloc", topk_ids, T, k, E, layout, align_or_max_m, payload,
                              payload_row_bytes, payload2, payload2_row_bytes, packed, packed2, rows_cap, counts,
                              seg_offsets, m_indices, output_index, dev_status, a);
  if (st) return st;
  const int64_t ws_need = route_workspace_bytes(a.R, E);
  if (ws_need > route_scratch_bytes())
    return fail(MOE_ERR_WORKSPACE,
                "moe_route_pack_noalloc: T*k=%d routes over E=%d experts need %lld scratch bytes, more than the "
                "library's fixed %lld; use moe_route_pack with a workspace",
                a.R, E, (long long)ws_need, (long long)route_scratch_bytes());
  if (ws_need > 0) {
    int32_t* ptr = nullptr;
    st = hip_status(route_scratch_ptr(&ptr), "moe_route_pack_noalloc: device address of the scratch array");
    if (st) return st;
    a.ws = ptr;
  }
  return hip_status(launch_route_pack(a, (hipStream_t)stream), "moe_route_pack_noalloc");
}

static moe_status check_gemm(const char* fn, int layout, const void* A, const void* W, const void* SW, void* D,
                             const int32_t* counts, const int32_t* seg_offsets, int E, int64_t rows_cap_or_max_m,
                             int N, int K) {
  if (layout != MOE_LAYOUT_CONTIGUOUS && layout != MOE_LAYOUT_MASKED)
    return fail(MOE_ERR_SHAPE, "%s: unknown layout %d", fn, layout);
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_SHAPE, "%s: E=%d must be in [1, %d]", fn, E, MOE_MAX_EXPERTS);
  if (N <= 0 || K <= 0 || rows_cap_or_max_m < 1)
    return fail(MOE_ERR_SHAPE, "%s: N=%d K=%d rows/max_m=%lld", fn, N, K, (long long)rows_cap_or_max_m);
  if (N % 128 || K % 128)
    return fail(MOE_ERR_UNSUPPORTED, "%s: N=%d and K=%d must be multiples of 128", fn, N, K);
  if (K / 128 > kMaxKBlocks) return fail(MOE_ERR_UNSUPPORTED, "%s: K=%d exceeds %d", fn, K, kMaxKBlocks * 128);
  const int64_t rows = layout == MOE_LAYOUT_MASKED ? (int64_t)E * rows_cap_or_max_m : rows_cap_or_max_m;
  if (rows > 0x7fffffff) return fail(MOE_ERR_SHAPE, "%s: too many rows", fn);
  if ((int64_t)N * K > 0xffffffffll) return fail(MOE_ERR_UNSUPPORTED, "%s: one expert's weights exceed 4 GiB", fn);
  if (!A || !W || !SW || !D || !counts) return fail(MOE_ERR_NULL, "%s: null pointer", fn);
  if (layout == MOE_LAYOUT_CONTIGUOUS && !seg_offsets)
    return fail(MOE_ERR_NULL, "%s: seg_offsets is required for the contiguous layout", fn);
  if (!aligned(A, 16) || !aligned(W, 16) || !aligned(D, 16))
    return fail(MOE_ERR_ALIGN, "%s: A, W and D must be 16-byte aligned", fn);
  return MOE_OK;
}

moe_status moe_grouped_gemm_fp8(int layout, const uint8_t* A, const float* SFA, const uint8_t* W, const float* SFW,
                                uint16_t* D, const int32_t* counts, const int32_t* seg_offsets, int E,
                                int64_t rows_cap_or_max_m, int N, int K, int expected_m, void* stream) {
  g_err[0] = 0;
  const int wpacked = (layout & MOE_WEIGHTS_PACKED) ? 1 : 0;
  layout &= ~MOE_WEIGHTS_PACKED;
  moe_status st = check_gemm("moe_grouped_gemm_fp8", layout, A, W, SFW, D, counts, seg_offsets, E, rows_cap_or_max_m,
                             N, K);
  if (st) return st;
  if (!SFA) return fail(MOE_ERR_NULL, "moe_grouped_gemm_fp8: SFA is null");
  if (!aligned(SFA, 4) || !aligned(SFW, 4)) return fail(MOE_ERR_ALIGN, "moe_grouped_gemm_fp8: scales misaligned");
  GemmArgs a{};
  a.A = A;
  a.SFA = SFA;
  a.W = W;
  a.SW = SFW;
  a.D = D;
  a.counts = counts;
  a.seg_offsets = seg_offsets;
  a.E = E;
  a.masked = layout == MOE_LAYOUT_MASKED;
  a.max_m = a.masked ? (int)rows_cap_or_max_m : 0;
  a.rows_cap = a.masked ? (int64_t)E * rows_cap_or_max_m : rows_cap_or_max_m;
  a.N = N;
  a.K = K;
  a.wpacked = wpacked;
  return hip_status(launch_gemm_fp8(a, expected_m, (hipStream_t)stream), "moe_grouped_gemm_fp8");
}

moe_status moe_grouped_gemm_fp8_swiglu(int layout, const uint8_t* A, const float* SFA, const uint8_t* W,
                                       const float* SFW, uint8_t* Q, float* SQ, const int32_t* counts,
                                       const int32_t* seg_offsets, int E, int64_t rows_cap_or_max_m, int I, int K,
                                       int expected_m, void* stream) {
  g_err[0] = 0;
  const int wpacked = (layout & MOE_WEIGHTS_PACKED) ? 1 : 0;
  layout &= ~MOE_WEIGHTS_PACKED;
  if (I <= 0 || I > 0x3fffffff) return fail(MOE_ERR_SHAPE, "moe_grouped_gemm_fp8_swiglu: I=%d", I);
  if (I % 128) return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_gemm_fp8_swiglu: I=%d is not a multiple of 128", I);
  moe_status st = check_gemm("moe_grouped_gemm_fp8_swiglu", layout, A, W, SFW, Q, counts, seg_offsets, E,
                             rows_cap_or_max_m, 2 * I, K);
  if (st) return st;
  if (!SFA || !SQ) return fail(MOE_ERR_NULL, "moe_grouped_gemm_fp8_swiglu: SFA or SQ is null");
  if (!aligned(SFW, 4) || !aligned(SQ, 4))
    return fail(MOE_ERR_ALIGN, "moe_grouped_gemm_fp8_swiglu: SFW and SQ must be 4-byte aligned");
  // the tall tile it runs on copies 4 K blocks of row scales per 16-byte load
  if ((K / 128) % 4)
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_gemm_fp8_swiglu: K=%d must be a multiple of 512", K);
  if (!aligned(SFA, 16)) return fail(MOE_ERR_ALIGN, "moe_grouped_gemm_fp8_swiglu: SFA must be 16-byte aligned");
  GemmArgs a{};
  a.A = A;
  a.SFA = SFA;
  a.W = W;
  a.SW = SFW;
  a.Q = Q;
  a.SQ = SQ;
  a.counts = counts;
  a.seg_offsets = seg_offsets;
  a.E = E;
  a.masked = layout == MOE_LAYOUT_MASKED;
  a.max_m = a.masked ? (int)rows_cap_or_max_m : 0;
  a.rows_cap = a.masked ? (int64_t)E * rows_cap_or_max_m : rows_cap_or_max_m;
  a.N = 2 * I;
  a.K = K;
  a.wpacked = wpacked;
  return hip_status(launch_gemm_fp8_swiglu(a, expected_m, (hipStream_t)stream), "moe_grouped_gemm_fp8_swiglu");
}

moe_status moe_grouped_gemm_int4(int layout, const uint16_t* A, const uint8_t* W4, const uint16_t* S16, uint16_t* D,
                                 const int32_t* counts, const int32_t* seg_offsets, int E, int64_t rows_cap_or_max_m,
                                 int N, int K, int expected_m, void* stream) {
  g_err[0] = 0;
  const int wpacked = (layout & MOE_WEIGHTS_PACKED) ? 1 : 0;
  layout &= ~MOE_WEIGHTS_PACKED;
  moe_status st = check_gemm("moe_grouped_gemm_int4", layout, A, W4, S16, D, counts, seg_offsets, E,
                             rows_cap_or_max_m, N, K);
  if (st) return st;
  if (!aligned(S16, 2)) return fail(MOE_ERR_ALIGN, "moe_grouped_gemm_int4: scales misaligned");
  // the packed kernel reads one lane's 4 scales of a group as one 8-byte load
  if (wpacked && !aligned(S16, 8))
    return fail(MOE_ERR_ALIGN, "moe_grouped_gemm_int4: packed scales must be 8-byte aligned");
  GemmArgs a{};
  a.A = (const uint8_t*)A;
  a.SFA = nullptr;
  a.W = W4;
  a.SW = S16;
  a.D = D;
  a.counts = counts;
  a.seg_offsets = seg_offsets;
  a.E = E;
  a.masked = layout == MOE_LAYOUT_MASKED;
  a.max_m = a.masked ? (int)rows_cap_or_max_m : 0;
  a.rows_cap = a.masked ? (int64_t)E * rows_cap_or_max_m : rows_cap_or_max_m;
  a.N = N;
  a.K = K;
  a.wpacked = wpacked;
  return hip_status(launch_gemm_int4(a, expected_m, (hipStream_t)stream), "moe_grouped_gemm_int4");
}

moe_status moe_pack_weight_bf16(const uint16_t* w, int E, int N, int K, uint16_t* packed, void* stream) {
  g_err[0] = 0;
  if (E < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_SHAPE, "moe_pack_weight_bf16: E=%d N=%d K=%d", E, N, K);
  if (N % 128 || K % 128)
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_weight_bf16: N=%d and K=%d must be multiples of 128", N, K);
  if ((int64_t)N * K * 2 > 0xffffffffll) return fail(MOE_ERR_UNSUPPORTED, "moe_pack_weight_bf16: one expert exceeds 4 GiB");
  if (E == 0) return MOE_OK;
  if (!w || !packed) return fail(MOE_ERR_NULL, "moe_pack_weight_bf16: null pointer");
  if (!aligned(w, 16) || !aligned(packed, 16))
    return fail(MOE_ERR_ALIGN, "moe_pack_weight_bf16: w and packed must be 16-byte aligned");
  const uint16_t* we = w + (int64_t)E * N * K;
  const uint16_t* pe = packed + (int64_t)E * N * K;
  if (w < pe && packed < we) return fail(MOE_ERR_SHAPE, "moe_pack_weight_bf16: w and packed overlap");
  // the bf16 bytes [E, N, 2K] in the FP8 fragment order with 2K bytes per row
  return hip_status(launch_pack_weight_fp8((const uint8_t*)w, E, N, 2 * K, (uint8_t*)packed, (hipStream_t)stream),
                    "moe_pack_weight_bf16");
}

moe_status moe_grouped_gemm_bf16(int layout, const uint16_t* A, const uint16_t* W, uint16_t* D,
                                 const int32_t* counts, const int32_t* seg_offsets, int E, int64_t rows_cap_or_max_m,
                                 int N, int K, int expected_m, void* stream) {
  g_err[0] = 0;
  const int wpacked = (layout & MOE_WEIGHTS_PACKED) ? 1 : 0;
  layout &= ~MOE_WEIGHTS_PACKED;
  moe_status st = check_gemm("moe_grouped_gemm_bf16", layout, A, W, W, D, counts, seg_offsets, E, rows_cap_or_max_m,
                             N, K);
  if (st) return st;
  if ((int64_t)N * K * 2 > 0xffffffffll)
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_gemm_bf16: one expert's weights exceed 4 GiB");
  GemmArgs a{};
  a.A = (const uint8_t*)A;
  a.SFA = nullptr;
  a.W = (const uint8_t*)W;
  a.SW = nullptr;
  a.D = D;
  a.counts = counts;
  a.seg_offsets = seg_offsets;
  a.E = E;
  a.masked = layout == MOE_LAYOUT_MASKED;
  a.max_m = a.masked ? (int)rows_cap_or_max_m : 0;
  a.rows_cap = a.masked ? (int64_t)E * rows_cap_or_max_m : rows_cap_or_max_m;
  a.N = N;
  a.K = K;
  a.wpacked = wpacked;
  return hip_status(launch_gemm_bf16(a, expected_m, (hipStream_t)stream), "moe_grouped_gemm_bf16");
}

moe_status moe_quant_weight_fp4(const uint16_t* w, int E, int N, int K, uint8_t* w4, uint8_t* sw, void* stream) {
  g_err[0] = 0;
  if (E < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_SHAPE, "moe_quant_weight_fp4: E=%d N=%d K=%d", E, N, K);
  if (K % 128) return fail(MOE_ERR_UNSUPPORTED, "moe_quant_weight_fp4: K=%d is not a multiple of 128", K);
  if (E == 0) return MOE_OK;
  if (!w || !w4 || !sw) return fail(MOE_ERR_NULL, "moe_quant_weight_fp4: null pointer");
  if (!aligned(w, 16) || !aligned(w4, 16))
    return fail(MOE_ERR_ALIGN, "moe_quant_weight_fp4: w and w4 must be 16-byte aligned");
  return hip_status(launch_quant_weight_fp4(w, E, N, K, w4, sw, (hipStream_t)stream), "moe_quant_weight_fp4");
}

moe_status moe_pack_weight_fp4(const uint8_t* w4, const uint8_t* sw, int E, int N, int K, uint8_t* w4_packed,
                               uint8_t* sw_packed, void* stream) {
  g_err[0] = 0;
  if (E < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_SHAPE, "moe_pack_weight_fp4: E=%d N=%d K=%d", E, N, K);
  if (N % 128 || K % 128)
    return fail(MOE_ERR_UNSUPPORTED, "moe_pack_weight_fp4: N=%d and K=%d must be multiples of 128", N, K);
  if ((int64_t)N * K / 2 > 0xffffffffll) return fail(MOE_ERR_UNSUPPORTED, "moe_pack_weight_fp4: one expert exceeds 4 GiB");
  if (E == 0) return MOE_OK;
  if (!w4 || !sw || !w4_packed || !sw_packed) return fail(MOE_ERR_NULL, "moe_pack_weight_fp4: null pointer");
  if (!aligned(w4, 16) || !aligned(w4_packed, 16) || !aligned(sw, 4) || !aligned(sw_packed, 4))
    return fail(MOE_ERR_ALIGN, "moe_pack_weight_fp4: codes must be 16-byte aligned, scales 4-byte aligned");
  const uint8_t* ranges[4][2] = {{w4, w4 + (int64_t)E * N * (K / 2)},
                                 {sw, sw + (int64_t)E * N * (K / 32)},
                                 {w4_packed, w4_packed + (int64_t)E * N * (K / 2)},
                                 {sw_packed, sw_packed + (int64_t)E * N * (K / 32)}};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if ((i >= 2 || j >= 2) && ranges[i][0] < ranges[j][1] && ranges[j][0] < ranges[i][1])
        return fail(MOE_ERR_SHAPE, "moe_pack_weight_fp4: an output overlaps another buffer");
  return hip_status(launch_pack_weight_fp4(w4, sw, E, N, K, w4_packed, sw_packed, (hipStream_t)stream),
                    "moe_pack_weight_fp4");
}

moe_status moe_grouped_gemm_fp8_fp4(int layout, const uint8_t* A, const float* SFA, const uint8_t* W4,
                                    const uint8_t* SW, uint16_t* D, const int32_t* counts,
                                    const int32_t* seg_offsets, int E, int64_t rows_cap_or_max_m, int N, int K,
                                    int expected_m, void* stream) {
  g_err[0] = 0;
  const int wpacked = (layout & MOE_WEIGHTS_PACKED) ? 1 : 0;
  layout &= ~MOE_WEIGHTS_PACKED;
  moe_status st = check_gemm("moe_grouped_gemm_fp8_fp4", layout, A, W4, SW, D, counts, seg_offsets, E,
                             rows_cap_or_max_m, N, K);
  if (st) return st;
  if (!SFA) return fail(MOE_ERR_NULL, "moe_grouped_gemm_fp8_fp4: SFA is null");
  if (!aligned(SFA, 4) || !aligned(SW, 4))
    return fail(MOE_ERR_ALIGN, "moe_grouped_gemm_fp8_fp4: SFA and SW must be 4-byte aligned");
  GemmArgs a{};
  a.A = A;
  a.SFA = SFA;
  a.W = W4;
  a.SW = SW;
  a.D = D;
  a.counts = counts;
  a.seg_offsets = seg_offsets;
  a.E = E;
  a.masked = layout == MOE_LAYOUT_MASKED;
  a.max_m = a.masked ? (int)rows_cap_or_max_m : 0;
  a.rows_cap = a.masked ? (int64_t)E * rows_cap_or_max_m : rows_cap_or_max_m;
  a.N = N;
  a.K = K;
  a.wpacked = wpacked;
  return hip_status(launch_gemm_fp4(a, expected_m, (hipStream_t)stream), "moe_grouped_gemm_fp8_fp4");
}

moe_status moe_quant_act_int8(const uint16_t* x, int64_t rows, int K, int8_t* q, float* s, void* stream) {
  g_err[0] = 0;
  if (rows < 0 || K <= 0) return fail(MOE_ERR_SHAPE, "moe_quant_act_int8: rows=%lld K=%d", (long long)rows, K);
  if (K % 128) return fail(MOE_ERR_UNSUPPORTED, "moe_quant_act_int8: K=%d is not a multiple of 128", K);
  if (rows == 0) return MOE_OK;
  if (!x || !q || !s) return fail(MOE_ERR_NULL, "moe_quant_act_int8: null pointer");
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4))
    return fail(MOE_ERR_ALIGN, "moe_quant_act_int8: x and q must be 16-byte aligned, s 4-byte aligned");
  return hip_status(launch_quant_int8(x, rows, K, 0, q, s, (hipStream_t)stream), "moe_quant_act_int8");
}

moe_status moe_quant_weight_int8(const uint16_t* w, int E, int N, int K, int8_t* q, float* sw, void* stream) {
  g_err[0] = 0;
  if (E < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_SHAPE, "moe_quant_weight_int8: E=%d N=%d K=%d", E, N, K);
  if (N % 128 || K % 128)
    return fail(MOE_ERR_UNSUPPORTED, "moe_quant_weight_int8: N=%d and K=%d must be multiples of 128", N, K);
  if (E == 0) return MOE_OK;
  if (!w || !q || !sw) return fail(MOE_ERR_NULL, "moe_quant_weight_int8: null pointer");
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(sw, 4))
    return fail(MOE_ERR_ALIGN, "moe_quant_weight_int8: w and q must be 16-byte aligned, sw 4-byte aligned");
  return hip_status(launch_quant_int8(w, (int64_t)E * N, K, N, q, sw, (hipStream_t)stream), "moe_quant_weight_int8");
}

moe_status moe_grouped_gemm_int8(int layout, const int8_t* A, const float* SA, const int8_t* W, const float* SW,
                                 uint16_t* D, const int32_t* counts, const int32_t* seg_offsets, int E,
                                 int64_t rows_cap_or_max_m, int N, int K, int expected_m, void* stream) {
  g_err[0] = 0;
  const int wpacked = (layout & MOE_WEIGHTS_PACKED) ? 1 : 0;
  layout &= ~MOE_WEIGHTS_PACKED;
  moe_status st = check_gemm("moe_grouped_gemm_int8", layout, A, W, SW, D, counts, seg_offsets, E, rows_cap_or_max_m,
                             N, K);
  if (st) return st;
  if (!SA) return fail(MOE_ERR_NULL, "moe_grouped_gemm_int8: SA is null");
  // a lane reads 4 consecutive weight scales of a K block as one 16-byte load
  if (!aligned(SA, 4) || !aligned(SW, 16))
    return fail(MOE_ERR_ALIGN, "moe_grouped_gemm_int8: SA must be 4-byte aligned, SW 16-byte aligned");
  GemmArgs a{};
  a.A = (const uint8_t*)A;
  a.SFA = SA;
  a.W = (const uint8_t*)W;
  a.SW = SW;
  a.D = D;
  a.counts = counts;
  a.seg_offsets = seg_offsets;
  a.E = E;
  a.masked = layout == MOE_LAYOUT_MASKED;
  a.max_m = a.masked ? (int)rows_cap_or_max_m : 0;
  a.rows_cap = a.masked ? (int64_t)E * rows_cap_or_max_m : rows_cap_or_max_m;
  a.N = N;
  a.K = K;
  a.wpacked = wpacked;
  return hip_status(launch_gemm_int8(a, expected_m, (hipStream_t)stream), "moe_grouped_gemm_int8");
}

moe_status moe_swiglu_quant(int layout, const uint16_t* gate_up, int64_t rows_cap_or_max_m, int I,
                            const int32_t* counts, const int32_t* seg_offsets, int E, uint8_t* q, float* sf,
                            void* stream) {
  g_err[0] = 0;
  if (layout != MOE_LAYOUT_CONTIGUOUS && layout != MOE_LAYOUT_MASKED)
    return fail(MOE_ERR_SHAPE, "moe_swiglu_quant: unknown layout %d", layout);
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_SHAPE, "moe_swiglu_quant: E=%d must be in [1, %d]", E,
                                                MOE_MAX_EXPERTS);
  if (I <= 0 || rows_cap_or_max_m < 1)
    return fail(MOE_ERR_SHAPE, "moe_swiglu_quant: I=%d rows/max_m=%lld", I, (long long)rows_cap_or_max_m);
  if (I % 128) return fail(MOE_ERR_UNSUPPORTED, "moe_swiglu_quant: I=%d is not a multiple of 128", I);
  const int64_t rows = layout == MOE_LAYOUT_MASKED ? (int64_t)E * rows_cap_or_max_m : rows_cap_or_max_m;
  if (rows > 0x7fffffff) return fail(MOE_ERR_SHAPE, "moe_swiglu_quant: too many rows");
  if (!gate_up || !counts || !q || !sf) return fail(MOE_ERR_NULL, "moe_swiglu_quant: null pointer");
  if (layout == MOE_LAYOUT_CONTIGUOUS && !seg_offsets)
    return fail(MOE_ERR_NULL, "moe_swiglu_quant: seg_offsets is required for the contiguous layout");
  if (!aligned(gate_up, 16) || !aligned(q, 16) || !aligned(sf, 4) || !aligned(counts, 4) ||
      (seg_offsets && !aligned(seg_offsets, 4)))
    return fail(MOE_ERR_ALIGN, "moe_swiglu_quant: gate_up and q must be 16-byte aligned, sf and tables 4-byte");
  SwigluArgs a;
  a.gu = gate_up;
  a.q = q;
  a.sf = sf;
  a.counts = counts;
  a.seg_offsets = seg_offsets;
  a.E = E;
  a.masked = layout == MOE_LAYOUT_MASKED;
  a.max_m = a.masked ? (int)rows_cap_or_max_m : 0;
  a.rows_cap = rows;
  a.I = I;
  return hip_status(launch_swiglu_quant(a, (hipStream_t)stream), "moe_swiglu_quant");
}

moe_status moe_unpermute_combine(const uint16_t* Y, int64_t y_rows, const int32_t* output_index,
                                 const float* topk_weights, int T, int k, int N, uint16_t* Z, void* stream) {
  g_err[0] = 0;
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || N <= 0 || y_rows < 0)
    return fail(MOE_ERR_SHAPE, "moe_unpermute_combine: T=%d k=%d N=%d y_rows=%lld", T, k, N, (long long)y_rows);
  if (N % 8) return fail(MOE_ERR_UNSUPPORTED, "moe_unpermute_combine: N=%d must be a multiple of 8", N);
  if (T == 0) return MOE_OK;
  if (!output_index || !topk_weights || !Z || (!Y && y_rows > 0))
    return fail(MOE_ERR_NULL, "moe_unpermute_combine: null pointer");
  if (!aligned(Z, 16) || (Y && !aligned(Y, 16)) || !aligned(output_index, 4) || !aligned(topk_weights, 4))
    return fail(MOE_ERR_ALIGN, "moe_unpermute_combine: Y and Z must be 16-byte aligned");
  return hip_status(launch_combine(Y, y_rows, output_index, topk_weights, T, k, N, Z, (hipStream_t)stream),
                    "moe_unpermute_combine");
}

int moe_stream_read_words(void) { return stream_read_grid(); }

moe_status moe_stream_read(const void* buf, int64_t bytes, uint32_t* out, void* stream) {
  g_err[0] = 0;
  if (bytes < 0 || bytes % 16)
    return fail(MOE_ERR_SHAPE, "moe_stream_read: bytes=%lld must be a multiple of 16", (long long)bytes);
  if (!out || (bytes && !buf)) return fail(MOE_ERR_NULL, "moe_stream_read: null pointer");
  if ((buf && !aligned(buf, 16)) || !aligned(out, 4))
    return fail(MOE_ERR_ALIGN, "moe_stream_read: buf must be 16-byte and out 4-byte aligned");
  return hip_status(launch_stream_read(buf, bytes, out, (hipStream_t)stream), "moe_stream_read");
}

}  // extern "C"
