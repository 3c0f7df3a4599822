// moe_device.h -- device helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kMaxExperts = 1024;
constexpr int kMaxKBlocks = 256;  // K <= 32768
constexpr int kWave = 64;

// ---------------------------------------------------------------- formats --
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest even (finite values; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Smallest e with amax <= 448 * 2^e, clamped to [-126, 127]; 0 when amax == 0.
// With amax = m * 2^x, m in [0.5, 1): 448 * 2^e = 0.875 * 2^(e+9), so
// e = x - 9 when m <= 0.875, else x - 8.  frexp is exact (denormals included).
__device__ __forceinline__ int pow2_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int x = __builtin_amdgcn_frexp_expf(amax);
  float m = __builtin_amdgcn_frexp_mantf(amax);
  int e = (m <= 0.875f) ? x - 9 : x - 8;
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

// fp32 power of two 2^e for e in [-126, 127] (a normal number).
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Round |v| <= 448 to the nearest OCP E4M3FN code, ties to even.  Exponent
// field 0 (|v| < 2^-6) is the subnormal range with step 2^-9; the sign is kept
// when the magnitude rounds to zero.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t s = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a < 0x3c800000u) {                      // |v| < 2^-6
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);  // 0..8, 8 == 0x08
  } else {
    uint32_t ex = (a >> 23) - 120u;           // biased E4M3 exponent, 1..15
    uint32_t man = a & 0x7fffffu;
    uint32_t keep = man >> 20, rest = man & 0xfffffu;
    uint32_t up = (rest > 0x80000u) | ((rest == 0x80000u) & keep);
    code = (ex << 3) + keep + up;             // a mantissa carry bumps the exponent
  }
  return code | s;
}

// ---------------------------------------------------------------- SwiGLU --
// silu(g) = g / (1 + exp(-g)) in fp32: x = -g log2(e) carried as hi + lo (hi the rounded product, lo its
// error by one fma plus g times the error of the fp32 log2(e)); t = exp2(hi) * (1 + lo ln 2) with the
// hardware exp2; silu = g * rcp(1 + t) with the hardware reciprocal.  Relative error a few fp32 ulps (about
// 3e-7); a gate below about -88 makes t infinite and the result -0, never NaN.
__device__ __forceinline__ float silu_f32(float g) {
  constexpr float kLog2e = 1.44269504088896341f;       // log2(e) rounded to fp32
  constexpr float kLog2eLo = 1.92596299e-08f;            // log2(e) - kLog2e
  constexpr float kLn2 = 0.693147180559945309f;
  const float hi = -g * kLog2e;
  const float lo = __builtin_fmaf(-g, kLog2e, -hi) - g * kLog2eLo;
  const float t = __builtin_amdgcn_exp2f(hi) * __builtin_fmaf(lo, kLn2, 1.0f);
  return g * __builtin_amdgcn_rcpf(1.0f + t);
}

// Maximum over each group of 8 (16) lanes, every lane of the group receiving it, by DPP moves inside the VALU
// (no LDS round trip): swap neighbours (quad_perm [1,0,3,2]), swap pairs ([2,3,0,1]), mirror each 8 lanes
// (row_half_mirror), and for 16 lanes mirror the 16 (row_mirror).  All lanes active.
__device__ __forceinline__ float max8_lanes(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
}
__device__ __forceinline__ float max16_lanes(float v) {
  v = max8_lanes(v);
  return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
}

// One 128-value block of SwiGLU and its 1x128 requantisation, spread over 16 consecutive lanes (all active):
// each lane holds 8 consecutive gate and up values as bf16 pairs (element 2i in the low half of word i),
// One 1x128 FP8 block held by 8 consecutive lanes, 16 consecutive bf16 per
// lane (raw0: elements 0..7, raw1: 8..15): the block's power-of-two exponent
// e (amax <= 448 * 2^e, smallest such e) and this lane's 16 E4M3 codes of
// x * 2^-e.  gfx950's v_cvt_pk_fp8_f32 converts to OCP E4M3FN with round to
// nearest even, subnormals and sign kept; the scaled values never exceed 448.
__device__ __forceinline__ uint4 fp8_block16(const v4i raw0, const v4i raw1, int& e) {
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
  e = pow2_exponent(amax);
  uint32_t o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(f[4 * r], -e),
                                           __builtin_amdgcn_ldexpf(f[4 * r + 1], -e), 0, false);
    c = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(f[4 * r + 2], -e),
                                       __builtin_amdgcn_ldexpf(f[4 * r + 3], -e), c, true);
    o[r] = (uint32_t)c;
  }
  return uint4{o[0], o[1], o[2], o[3]};
}

// h = silu(gate) * up in fp32, the block's amax over the 16 lanes, e = pow2_exponent(amax), and this lane's
// 8 E4M3 codes of h * 2^-e (round to nearest even) packed little-endian into *codes.  Returns e.
__device__ __forceinline__ int swiglu_quant16(const v4i g, const v4i u, uint2* codes) {
  float h[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t gw = (uint32_t)g[i], uw = (uint32_t)u[i];
    h[2 * i] = silu_f32(bf16_to_f32(gw & 0xffffu)) * bf16_to_f32(uw & 0xffffu);
    h[2 * i + 1] = silu_f32(bf16_to_f32(gw >> 16)) * bf16_to_f32(uw >> 16);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(h[i]));
  amax = max16_lanes(amax);
  const int e = pow2_exponent(amax);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = __builtin_amdgcn_ldexpf(h[i], -e);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
  codes->x = (uint32_t)lo;
  codes->y = (uint32_t)hi;
  return e;
}

// ----------------------------------------------------------- compile time --
template <int V>
struct IntC {
  static constexpr int value = V;
};
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

// ------------------------------------------------------------------ waves --
// Mark a wave-uniform value as such (keeps it in an SGPR).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

// LDS byte offset of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// Direct global -> LDS copies: lane i of the wave writes lds_base + 16*i (or
// 4*i); lds_base must be wave-uniform.  Issued through inline asm on purpose:
// the compiler cannot tell which LDS bytes such a copy writes and would wait
// for every outstanding load before any LDS read.  Callers own the vmcnt
// accounting (wait_vmcnt) and the barrier that publishes the data.
__device__ __forceinline__ void dma16(const void* gsrc, const void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds_base));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gsrc), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* gsrc, const void* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds_base));
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(gsrc), "{m0}"(m0) : "memory");
}

// Workgroup barrier that publishes this wave's LDS writes but, unlike
// __syncthreads(), does not wait for outstanding global loads (prefetches).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// ------------------------------------------------------------ block scan --
// Exclusive prefix sum of v[0..n) in LDS, in place; v[n] receives the total.
// All threads of the block must call it.  n <= 4 * blockDim.x.
__device__ inline void block_exclusive_scan(int* v, int n, int* tmp /* >= blockDim.x + 1 ints */) {
  const int tid = threadIdx.x, nt = blockDim.x;
  int per = (n + nt - 1) / nt;
  int lo = tid * per, hi = min(lo + per, n);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += v[i];
  tmp[tid] = local;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    int add = (tid >= off) ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  int run = tmp[tid] - local;  // exclusive prefix of this thread's range
  if (tid == nt - 1) tmp[nt] = tmp[tid];
  __syncthreads();
  for (int i = lo; i < hi; ++i) {
    int x = v[i];
    v[i] = run;
    run += x;
  }
  if (tid == 0) v[n] = tmp[nt];
  __syncthreads();
}

// Index of the last e in [0, n) with pre[e] <= x (pre non-decreasing, pre[0] <= x).
__device__ __forceinline__ int upper_bound_minus1(const int* pre, int n, int x) {
  int lo = 0, hi = n;  // answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (pre[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace moe
