// quant.hip -- FP8 1x128 / 128x128 power-of-two quantisation, INT8 (1, 1, 128)
// quantisation and the group-128 4-bit weight format.
//
// FP8 rule (nxmr.cn DeepGEMM FP8 article, "补偿机制一"): each block's scale is an
// exact power of two, amax/448 rounded up, so scaling is an exponent shift and
// no scaled value exceeds the E4M3 range of 448.  Codes are round-to-nearest-
// even E4M3FN of x * 2^-e.
//
// INT4 format (ONNX Runtime "MatMulNBits -- CUDA Operator Documentation",
// sec. 2): per output row n, K/2 bytes with two 4-bit weights per byte (low
// nibble = even k), one fp16 scale per 128 along K, value (q - 8) * scale.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// One 8-lane group per 128-element block: lane holds 16 consecutive bf16 (two
// 16-byte loads) and stores their 16 codes with one 16-byte store.  A wave
// covers 8 blocks per pass.  HBM-bound; ordinary loads (nontemporal ones,
// 16-lane groups with 8-byte stores and deeper per-wave batches all measured
// slower on 4096 x 7168 and 8192 x 4096).
__device__ __forceinline__ void quant_act_block(const v4i raw0, const v4i raw1, int64_t blk, bool ok, int sub,
                                                uint8_t* __restrict__ q, float* __restrict__ sf) {
  int e;
  const uint4 codes = fp8_block16(raw0, raw1, e);
  if (ok) {
    *(uint4*)(q + blk * 128 + sub * 16) = codes;
    if (sub == 0) sf[blk] = pow2f(e);
  }
}

__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int64_t nblocks, int kb,
                                                         uint8_t* __restrict__ q, float* __restrict__ sf) {
  const int lane = lane_id();
  const int sub = lane & 7;
  const int64_t gwave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t b0 = gwave * 8; b0 < nblocks; b0 += nwaves * 8) {
    const int64_t blk = b0 + (lane >> 3);
    const bool ok = blk < nblocks;
    v4i r0 = {0, 0, 0, 0}, r1 = {0, 0, 0, 0};
    if (ok) {
      r0 = *(const v4i*)(x + blk * 128 + sub * 16);
      r1 = *(const v4i*)(x + blk * 128 + sub * 16 + 8);
    }
    quant_act_block(r0, r1, blk, ok, sub, q, sf);
  }
}

// One workgroup (256 threads) per 128x128 weight block; each thread holds 64
// elements (8 rows x 8 consecutive k).
__global__ __launch_bounds__(256) void quant_weight_fp8_kernel(const uint16_t* __restrict__ w, int N, int K,
                                                                uint8_t* __restrict__ q, float* __restrict__ sfw) {
  __shared__ float s_red[4];
  const int nb = N / 128, kb = K / 128;
  const int64_t blk = blockIdx.x;  // (e, nb, kb) flattened
  const int kbi = (int)(blk % kb);
  const int nbi = (int)((blk / kb) % nb);
  const int64_t e = blk / ((int64_t)kb * nb);
  const int tid = threadIdx.x;
  const int col = (tid & 15) * 8;        // k offset within the block
  const int row0 = tid >> 4;             // 0..15; rows row0 + 16*j
  const int64_t base = (e * N + (int64_t)nbi * 128) * K + (int64_t)kbi * 128 + col;
  float f[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v4i raw = *(const v4i*)(w + base + (int64_t)(row0 + 16 * j) * K);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t u = (uint32_t)raw[i];
      f[j][2 * i] = bf16_to_f32(u & 0xffffu);
      f[j][2 * i + 1] = bf16_to_f32(u >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(f[j][2 * i]), fabsf(f[j][2 * i + 1])));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if (lane_id() == 0) s_red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const int ex = pow2_exponent(amax);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= e4m3_encode(__builtin_amdgcn_ldexpf(f[j][i], -ex)) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= e4m3_encode(__builtin_amdgcn_ldexpf(f[j][4 + i], -ex)) << (8 * i);
    uint2 out;
    out.x = lo;
    out.y = hi;
    *(uint2*)(q + base + (int64_t)(row0 + 16 * j) * K) = out;
  }
  if (tid == 0) sfw[blk] = pow2f(ex);
}

// One 16-lane group per (row n, 128-group): lane holds 8 consecutive weights.
__global__ __launch_bounds__(256) void quant_weight_int4_kernel(const uint16_t* __restrict__ w, int64_t ngroups,
                                                                 uint8_t* __restrict__ q4,
                                                                 uint16_t* __restrict__ s16) {
  const int lane = lane_id();
  const int sub = lane & 15;
  const int64_t gwave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t g0 = gwave * 4; g0 < ngroups; g0 += nwaves * 4) {
    const int64_t g = g0 + (lane >> 4);
    const bool ok = g < ngroups;
    v4i raw = {0, 0, 0, 0};
    if (ok) raw = *(const v4i*)(w + g * 128 + sub * 8);
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t u = (uint32_t)raw[i];
      f[2 * i] = bf16_to_f32(u & 0xffffu);
      f[2 * i + 1] = bf16_to_f32(u >> 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    // s = fp16(amax / 7) with the division in fp32 (correctly rounded) and the
    // conversion to fp16 round-to-nearest-even; guards for 0, underflow, overflow.
    _Float16 h;
    if (amax == 0.0f) {
      h = (_Float16)1.0f;
    } else {
      float s32 = amax / 7.0f;
      h = (_Float16)s32;
      if ((float)h == 0.0f) h = (_Float16)5.9604644775390625e-08f;  // 2^-24
      if (!((float)h <= 65504.0f)) h = (_Float16)65504.0f;
    }
    const float s = (float)h;
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float qf = __builtin_rintf(f[i] / s) + 8.0f;
      qf = fminf(fmaxf(qf, 0.0f), 15.0f);
      packed |= ((uint32_t)qf) << (4 * i);
    }
    if (ok) {
      *(uint32_t*)(q4 + g * 64 + sub * 4) = packed;
      if (sub == 0) s16[g] = __builtin_bit_cast(uint16_t, h);
    }
  }
}

// Fragment-packed FP8 weight order (the layout moe_pack_weight_fp8 defines):
// one thread per 16-byte output chunk.  Output chunk r of an expert is lane
// L = r % 64 of half h = (r / 64) % 2 of the 2-KB block b = r / 128, with
// b = kb * (N/16) + cb; it holds bytes 128kb + 64h + 16(L/16) .. +15 of weight
// column 16cb + L % 16.  Stores are contiguous; each load reads 16 bytes of a
// row (a permutation, HBM-bound, run once when weights are prepared).
__global__ __launch_bounds__(256) void pack_weight_fp8_kernel(const uint8_t* __restrict__ q, int64_t chunks,
                                                              int64_t expert_chunks, int N, int K,
                                                              uint8_t* __restrict__ out) {
  const int ncb = N / 16;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = c / expert_chunks;
    const int64_t r = c - e * expert_chunks;
    const int64_t b = r >> 7;
    const int qq = (int)(r & 127);
    const int h = qq >> 6, L = qq & 63;
    const int64_t kb = b / ncb;
    const int cb = (int)(b - kb * ncb);
    const int64_t n = 16 * cb + (L & 15);
    const int64_t k = 128 * kb + 64 * h + 16 * (L >> 4);
    const v4i v = *(const v4i*)(q + (e * N + n) * K + k);
    *(v4i*)(out + c * 16) = v;
  }
}

// Fragment-packed 4-bit weight order (moe_pack_weight_int4): one thread per
// 16-byte output chunk.  Output chunk r of an expert is lane L = r % 64 of the
// 1-KB block b = r / 64 = g * (N/16) + cb: column 16cb + L % 16, and for each
// dword d the 8 weights k0 = 128g + 8(4d + L/16) .. k0 + 7, whose MatMulNBits
// bytes are one source dword s.  The even k (low nibbles of s) fill the low
// half of the output dword, the odd k (high nibbles) the high half.
__device__ __forceinline__ uint32_t gather_nibbles(uint32_t x) {  // low nibbles of the 4 bytes -> 16 bits
  x &= 0x0F0F0F0Fu;
  return (x & 0xFu) | ((x >> 4) & 0xF0u) | ((x >> 8) & 0xF00u) | ((x >> 12) & 0xF000u);
}
__global__ __launch_bounds__(256) void pack_weight_int4_kernel(const uint8_t* __restrict__ q4, int64_t chunks,
                                                               int64_t expert_chunks, int N, int K,
                                                               uint8_t* __restrict__ out) {
  const int ncb = N / 16;
  const int64_t rowb = K / 2;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = c / expert_chunks;
    const int64_t r = c - e * expert_chunks;
    const int64_t b = r >> 6;
    const int L = (int)(r & 63);
    const int64_t g = b / ncb;
    const int cb = (int)(b - g * ncb);
    const int64_t n = 16 * cb + (L & 15);
    const uint8_t* src = q4 + (e * N + n) * rowb + 64 * g + 4 * (L >> 4);
    v4i v;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t sw = *(const uint32_t*)(src + 16 * d);  // k0 = 128g + 8(4d + h): byte 64g + 16d + 4h
      v[d] = (int)(gather_nibbles(sw) | (gather_nibbles(sw >> 4) << 16));
    }
    *(v4i*)(out + c * 16) = v;
  }
}

// Packed scale order: element i of an expert's [K/128][N/64][16][4] block.
__global__ __launch_bounds__(256) void pack_scale_int4_kernel(const uint16_t* __restrict__ s16, int64_t total,
                                                              int64_t per_expert, int N, int KG,
                                                              uint16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i / per_expert;
    int64_t r = i - e * per_expert;
    const int cb = (int)(r & 3);
    const int c16 = (int)((r >> 2) & 15);
    r >>= 6;
    const int64_t n64 = r % (N / 64), g = r / (N / 64);
    const int64_t n = 64 * n64 + 16 * cb + c16;
    out[i] = s16[(e * N + n) * KG + g];
  }
}

// INT8 (1, 1, 128) blocks (AsymGEMM README, "API Reference", INT8 asymmetric
// GEMM: int8 data with one fp32 scale per row and 128 elements along K).
// Symmetric rule: s = amax / 127 (fp32, correctly rounded), codes
// rne(x / s) clamped to +-127, s = 1 for an all-zero block.  The division is
// the correctly rounded fp32 one (hipcc's default for '/'), since it decides
// the integer code.  One 8-lane group per block, lane holds 16 consecutive
// elements, as for the FP8 activation codes.  The scales are written
// [rows, K/128] for activations and in the K-block-major [E, K/128, N] order
// for weights (the order the grouped GEMM reads them in).
__device__ __forceinline__ void quant_int8_block(const v4i raw0, const v4i raw1, bool ok, int sub,
                                                 int8_t* __restrict__ qblk, float* __restrict__ sfp) {
  float f[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w0 = (uint32_t)raw0[i], w1 = (uint32_t)raw1[i];
    f[2 * i] = bf16_to_f32(w0 & 0xffffu);
    f[2 * i + 1] = bf16_to_f32(w0 >> 16);
    f[8 + 2 * i] = bf16_to_f32(w1 & 0xffffu);
    f[8 + 2 * i + 1] = bf16_to_f32(w1 >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = max8_lanes(amax);
  const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
  // The code is rne of the correctly rounded quotient x / s.  y = x * rn(1/s)
  // is within 1.5 * 2^-16 of that quotient (two roundings of relative size
  // 2^-24 each, |x / s| <= 127 * (1 + 2^-23)), so rint(y) is the same code
  // unless a half-integer lies within 2^-15 of y; those rare elements, and
  // every element of a block whose scale is below 2^-100 (its reciprocal may
  // not be a normal fp32 number), take the division itself.
  const float rs = 1.0f / s;
  const bool fast = s >= 0x1p-100f;
  uint32_t o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = f[4 * r + i];
      const float y = x * rs;
      float q = __builtin_rintf(y);
      if (!(fast && fabsf(y - (floorf(y) + 0.5f)) > 0x1p-15f)) q = __builtin_rintf(x / s);
      const float c = fminf(fmaxf(q, -127.0f), 127.0f);
      w |= ((uint32_t)(int)c & 0xffu) << (8 * i);
    }
    o[r] = w;
  }
  if (ok) {
    *(uint4*)(qblk + sub * 16) = uint4{o[0], o[1], o[2], o[3]};
    if (sub == 0) *sfp = s;
  }
}

// Activations: block b = row * kb + j; scale at sf[b].  Weights (wn > 0):
// row = e * wn + n, scale at sf[(e * kb + j) * wn + n].
__global__ __launch_bounds__(256) void quant_int8_kernel(const uint16_t* __restrict__ x, int64_t nblocks, int kb,
                                                         int wn, int8_t* __restrict__ q, float* __restrict__ sf) {
  const int lane = lane_id();
  const int sub = lane & 7;
  const int64_t gwave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t b0 = gwave * 8; b0 < nblocks; b0 += nwaves * 8) {
    const int64_t blk = b0 + (lane >> 3);
    const bool ok = blk < nblocks;
    v4i r0 = {0, 0, 0, 0}, r1 = {0, 0, 0, 0};
    if (ok) {
      r0 = *(const v4i*)(x + blk * 128 + sub * 16);
      r1 = *(const v4i*)(x + blk * 128 + sub * 16 + 8);
    }
    int64_t si = blk;
    if (wn > 0) {
      const int64_t row = blk / kb, j = blk - row * kb;
      const int64_t e = row / wn, n = row - e * wn;
      si = (e * kb + j) * wn + n;
    }
    quant_int8_block(r0, r1, ok, sub, q + blk * 128, sf + (ok ? si : 0));
  }
}

static int grid_for(int64_t work_items, int per_block, int cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

hipError_t launch_quant_act(const uint16_t* x, int64_t rows, int K, uint8_t* q, float* sf, hipStream_t s) {
  const int64_t nblocks = rows * (K / 128);
  if (nblocks == 0) return hipSuccess;
  const int grid = grid_for(nblocks, 32, device_info().cus * 16);  // 32 blocks per 256-thread WG per pass
  quant_act_kernel<<<grid, 256, 0, s>>>(x, nblocks, K / 128, q, sf);
  return hipGetLastError();
}

hipError_t launch_quant_int8(const uint16_t* x, int64_t rows, int K, int wn, int8_t* q, float* sf, hipStream_t s) {
  const int64_t nblocks = rows * (K / 128);
  if (nblocks == 0) return hipSuccess;
  const int grid = grid_for(nblocks, 32, device_info().cus * 16);  // 32 blocks per 256-thread WG per pass
  quant_int8_kernel<<<grid, 256, 0, s>>>(x, nblocks, K / 128, wn, q, sf);
  return hipGetLastError();
}

hipError_t launch_quant_weight_fp8(const uint16_t* w, int E, int N, int K, uint8_t* q, float* sfw, hipStream_t s) {
  const int64_t nblocks = (int64_t)E * (N / 128) * (K / 128);
  if (nblocks == 0) return hipSuccess;
  if (nblocks > 0x7fffffff) return hipErrorInvalidValue;
  quant_weight_fp8_kernel<<<(unsigned)nblocks, 256, 0, s>>>(w, N, K, q, sfw);
  return hipGetLastError();
}

hipError_t launch_pack_weight_fp8(const uint8_t* q, int E, int N, int K, uint8_t* packed, hipStream_t s) {
  const int64_t expert_chunks = (int64_t)N * K / 16;
  const int64_t chunks = (int64_t)E * expert_chunks;
  if (chunks == 0) return hipSuccess;
  const int grid = grid_for(chunks, 256, device_info().cus * 8);
  pack_weight_fp8_kernel<<<grid, 256, 0, s>>>(q, chunks, expert_chunks, N, K, packed);
  return hipGetLastError();
}

hipError_t launch_pack_weight_int4(const uint8_t* q4, const uint16_t* s16, int E, int N, int K, uint8_t* q4_packed,
                                   uint16_t* s16_packed, hipStream_t s) {
  const int64_t expert_chunks = (int64_t)N * K / 32;
  const int64_t chunks = (int64_t)E * expert_chunks;
  if (chunks == 0) return hipSuccess;
  pack_weight_int4_kernel<<<grid_for(chunks, 256, device_info().cus * 8), 256, 0, s>>>(q4, chunks, expert_chunks, N, K,
                                                                                       q4_packed);
  const int64_t per_expert = (int64_t)N * (K / 128), total = (int64_t)E * per_expert;
  pack_scale_int4_kernel<<<grid_for(total, 256, device_info().cus * 8), 256, 0, s>>>(s16, total, per_expert, N, K / 128,
                                                                                     s16_packed);
  return hipGetLastError();
}

hipError_t launch_quant_weight_int4(const uint16_t* w, int E, int N, int K, uint8_t* q4, uint16_t* s16,
                                    hipStream_t s) {
  const int64_t ngroups = (int64_t)E * N * (K / 128);
  if (ngroups == 0) return hipSuccess;
  const int grid = grid_for(ngroups, 16, device_info().cus * 16);
  quant_weight_int4_kernel<<<grid, 256, 0, s>>>(w, ngroups, q4, s16);
  return hipGetLastError();
}

}  // namespace moe
