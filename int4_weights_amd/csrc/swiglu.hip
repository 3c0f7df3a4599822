// swiglu.hip -- moe_swiglu_quant: SwiGLU on the up-projection's packed rows and
// the 1x128 FP8 requantisation the down-projection reads.
//
// h[p, j] = silu(gate[p, j]) * up[p, j],  gate = columns 0..I-1, up = I..2I-1
// of the up-projection output (the fused gate+up expert weight of a
// DeepSeek-V3-shaped layer is 2 x 2048 columns; CuTeDSL bei Perplexity lists
// activation kernels among the MoE kernels), then per row and 128-column block
// the power-of-two scale 2^e with e the smallest integer with amax <= 448 * 2^e
// and the E4M3 codes of h * 2^-e (nxmr.cn DeepGEMM FP8 article, "补偿机制一").
// h is quantised as computed in fp32, never rounded to bf16 in between.
//
// fp32 evaluation (swiglu_quant16, shared with the up-projection GEMM that
// fuses this step): g, u exact from bf16, silu_f32(g) * u; relative error a
// few fp32 ulps (about 3e-7) against the exact value.
//
// Only the rows of the segments are touched (counts clipped to the segment
// capacity, as in the grouped GEMM): padding rows are neither read nor
// written.  Each workgroup puts the exclusive prefix of the valid rows per
// expert in LDS, so the i-th valid row maps to its packed row by a binary
// search; 16 lanes handle one row at a time (16 bytes of gate and 16 of up
// per lane and 128-column block, kSwQ blocks of loads in flight), a wave 4
// rows.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kSwQ = 6;  // 128-column blocks of loads in flight per lane

__global__ __launch_bounds__(256) void swiglu_quant_kernel(const SwigluArgs a) {
  __shared__ int s_cum[kMaxExperts + 1];
  __shared__ int s_start[kMaxExperts];
  __shared__ int s_tmp[257];
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
    int r = a.counts[e];
    int64_t st, cap;
    if (a.masked) {
      st = (int64_t)e * a.max_m;
      cap = a.max_m;
    } else {
      st = a.seg_offsets[e];
      cap = (st >= 0 && st < a.rows_cap) ? a.rows_cap - st : 0;
    }
    if (r < 0) r = 0;
    if (r > cap) r = (int)cap;
    s_cum[e] = r;
    s_start[e] = (int)st;
  }
  __syncthreads();
  block_exclusive_scan(s_cum, a.E, s_tmp);  // s_cum[E] = valid rows in all
  const int ib = a.I / 128;
  const int nrows = s_cum[a.E];
  const int lane = lane_id(), sub = lane & 15;
  const int gwave = (int)(((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int nwaves = (int)(((int64_t)gridDim.x * blockDim.x) >> 6);
  const int64_t rs = 2 * (int64_t)a.I;  // bf16 elements per gate_up row
  // each 16-lane group takes one valid row at a time and walks its 128-column blocks, kSwQ blocks of loads in
  // flight; the row's packed position is found once
  for (int vr0 = gwave * 4; vr0 < nrows; vr0 += nwaves * 4) {
    const int vr = vr0 + (lane >> 4);
    const bool rok = vr < nrows;
    int64_t p = 0;
    if (rok) {
      const int e = upper_bound_minus1(s_cum, a.E + 1, vr);  // last e with s_cum[e] <= vr (< E: vr < nrows)
      p = s_start[e] + (vr - s_cum[e]);
    }
    const uint16_t* src = a.gu + p * rs + sub * 8;
    uint8_t* qrow = a.q + p * a.I + sub * 8;
    float* sfrow = a.sf + p * ib;
    for (int kb0 = 0; kb0 < ib; kb0 += kSwQ) {
      v4i g[kSwQ], u[kSwQ];
#pragma unroll
      for (int j = 0; j < kSwQ; ++j) {
        if (rok && kb0 + j < ib) {
          // read once: streamed past the caches
          g[j] = __builtin_nontemporal_load((const v4i*)(src + (kb0 + j) * 128));
          u[j] = __builtin_nontemporal_load((const v4i*)(src + (kb0 + j) * 128 + a.I));
        } else {
          g[j] = v4i{0, 0, 0, 0};
          u[j] = v4i{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int j = 0; j < kSwQ; ++j) {
        uint2 o;
        const int e = swiglu_quant16(g[j], u[j], &o);
        if (rok && kb0 + j < ib) {
          *(uint2*)(qrow + (kb0 + j) * 128) = o;
          if (sub == 0) sfrow[kb0 + j] = pow2f(e);
        }
      }
    }
  }
}

hipError_t launch_swiglu_quant(const SwigluArgs& a, hipStream_t s) {
  // the valid rows are known on the device only: size the grid for the segments' capacity (16 rows per
  // workgroup and pass), at most 8 workgroups per CU so that each one's prologue is paid about once per CU slot
  int64_t grid = (a.rows_cap + 15) / 16;
  const int64_t cap = (int64_t)device_info().cus * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  swiglu_quant_kernel<<<(unsigned)grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
