// gemm_int4.hip -- 4-bit weight-only grouped GEMM for gfx950.
//
// D[p, n] = bf16( sum_g s[e,n,g] * sum_{k in g} a[p,k] * (q[e,n,k] - 8) )
// (ONNX Runtime "MatMulNBits -- CUDA Operator Documentation", sec. 2 "Weight
// Format": row n is K/2 bytes, two 4-bit weights per byte, one scale per
// 128-element group along K, symmetric zero point 8; sec. 4.1 describes a
// warp-per-column GEMV for one token -- prior art for NVIDIA, not used here.)
//
// Design for CDNA4 (decode-sized segments: a handful of rows per expert):
//  * Same persistent per-expert unit scheduler as the FP8 GEMM; a unit is
//    (expert, 256 columns, up to 16*RB rows).  Each wave owns 64 columns.
//  * The 4-bit weights stream from HBM into VGPRs through an S-deep ring: one
//    16-byte load per lane covers 32 k of one column.
//  * Dequantisation costs one AND-OR per two weights: OR-ing the nibble into
//    the mantissa of bf16 128.0 (0x4300) gives 128 + q exactly.  The bf16
//    matrix instruction v_mfma_f32_16x16x32_bf16 multiplies it with the
//    activations, and one extra instruction per group against the constant
//    -136 adds -136 * sum(a), so the group partial is exactly
//    sum a * (128 + q) - 136 * sum a = sum a * (q - 8) up to fp32 rounding.
//    The correction is shared by all column blocks of the wave.
//  * The nibble pairs land as (k, k+4) within each 8-k run; the activation
//    fragment is permuted the same way (dot products are invariant under a
//    common permutation of k).
//  * Per-group fp16 scales are applied to the fp32 group partial by one FMA;
//    the accumulator layout gives each lane one column, hence one scale.
//  * Activations are staged in LDS (two slots, XOR-swizzled) from VGPR-ring
//    loads, as in the FP8 kernel.
//
// Weights in the packed order (moe_pack_weight_int4) take a second kernel
// built for decode, where each expert holds a handful of rows and the kernel
// is bound by the weight stream:
//  * the four waves of a workgroup share nothing but the unit table: each
//    streams its own 64 columns with no barrier, so a late load stalls one
//    wave only;
//  * each dword of the packed order holds 8 consecutive k with k + 2i and
//    k + 2i + 1 at nibbles i and i + 4, so the dequantised pairs are in
//    natural order and the activation fragment is used as loaded: 16 bytes
//    per matrix instruction, read straight from global memory (the rows of an
//    expert stay in L2 for its column tiles);
//  * the packed scales put the 4 column blocks of one lane's column next to
//    each other: one 8-byte load per lane and K group, in the weight ring.
#include "gemm_common.h"

namespace moe {

template <int RB, int S>
struct I4Cfg {
  static constexpr int BM = 16 * RB;
  static constexpr int kApw = RB;            // 16-byte A loads per lane per stage (4 rows of 256 B)
  static constexpr int kAStage = BM * 256;   // bytes per LDS slot
  // K groups whose scales are held in LDS at once (a power of two); a longer K
  // restages them every kScG groups
  static constexpr int kScG = RB == 1 ? kMaxKBlocks : kMaxKBlocks / 2;
};

template <int RB, int S>
struct I4Smem {
  uint8_t a[2][I4Cfg<RB, S>::kAStage];
  uint16_t sc[I4Cfg<RB, S>::kScG][kBN];  // group scales (fp16) of the unit, [group mod kScG][column of the N tile]
};

__device__ __forceinline__ v8bf as_bf(const v4i& x) { return __builtin_bit_cast(v8bf, x); }

template <int RB, int S>
__device__ __forceinline__ void int4_unit(const GemmArgs& a, const Unit& u, I4Smem<RB, S>& sm, int wv, int lane) {
  using C = I4Cfg<RB, S>;
  const int l16 = lane & 15, lg = lane >> 4;
  const int K = a.K, N = a.N, KG = K / 128;
  const int ncol0 = u.n0 + 64 * wv;
  const bool wave_on = ncol0 < N;

  // 4-bit weights, MatMulNBits order: column n's group g is 64 bytes at n*K/2 + 64g
  const uint8_t* wbase = a.W + (int64_t)u.e * N * (K / 2);
  uint32_t woff[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    int n = ncol0 + 16 * cb + l16;
    if (n >= N) n = N - 1;
    woff[cb] = (uint32_t)n * (uint32_t)(K / 2) + 16u * lg;
  }
  // the unit's group scales: its columns' rows of S16 are one contiguous block
  // (kBN x KG halves); groups gb .. gb+kScG-1 are staged into LDS
  // [group][column] with a batch of coalesced loads
  const uint16_t* sblk = (const uint16_t*)a.SW + ((int64_t)u.e * N + u.n0) * KG;
  const int scols = min(kBN, N - u.n0);
  auto stage_scales = [&](int gb) {
    const int cnt = min(C::kScG, KG - gb), total = scols * cnt;
    const float inv = 1.0f / (float)cnt;
    for (int base = threadIdx.x; base < total; base += 256 * 16) {
      uint16_t v[16];
      int col[16], grp[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int idx = base + 256 * i;
        int c = (int)(((float)idx + 0.5f) * inv);  // idx / cnt, corrected to be exact below
        int g = idx - c * cnt;
        if (g < 0) { --c; g += cnt; }
        if (g >= cnt) { ++c; g -= cnt; }
        col[i] = c;
        grp[i] = g;
        v[i] = idx < total ? sblk[(int64_t)c * KG + gb + g] : (uint16_t)0;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (base + 256 * i < total) sm.sc[grp[i]][col[i]] = v[i];
    }
  };
  stage_scales(0);  // the previous unit ended with a barrier
  int scol[4];  // this lane's columns within the N tile (clamped for an idle wave)
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) scol[cb] = min(64 * wv + 16 * cb + l16, min(kBN, N - u.n0) - 1);
  const uint8_t* abase = a.A + (int64_t)u.row0 * K * 2;
  uint32_t aoff[C::kApw];
#pragma unroll
  for (int i = 0; i < C::kApw; ++i) {
    const int q = wv * C::kApw + i;            // 1 KB block of the stage (4 rows)
    const int r = 4 * q + (lane >> 4);         // tile row written by this lane
    const int c = (lane & 15) ^ (r & 15);      // 16-byte chunk that lands at position lane & 15
    aoff[i] = (uint32_t)min(r, u.mrows - 1) * (uint32_t)(K * 2) + 16u * c;
  }

  v4i wq[S][4];
  v4i ar[S][C::kApw];
  v4f acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int ks_req, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const int ks = min(ks_req, KG - 1);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) wq[slot][cb] = *(const v4i*)(wbase + (woff[cb] + (uint32_t)ks * 64u));
#pragma unroll
    for (int i = 0; i < C::kApw; ++i) ar[slot][i] = *(const v4i*)(abase + (aoff[i] + (uint32_t)ks * 256u));
  };

  auto commit = [&](int ks, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    uint8_t* dst = &sm.a[ks & 1][0];
#pragma unroll
    for (int i = 0; i < C::kApw; ++i) *(v4i*)(dst + (wv * C::kApw + i) * 1024 + 16 * lane) = ar[slot][i];
  };

  // activation fragment reads: row m = 16*rb + l16 at m*256, chunk c at c ^ l16
  int aoff_rd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff_rd[i] = l16 * 256 + 16 * ((4 * lg + i) ^ l16);
  const v4i kNeg136 = v4i{(int)0xC308C308u, (int)0xC308C308u, (int)0xC308C308u, (int)0xC308C308u};
  // The nibble mask and the bf16 bias live in registers the compiler cannot
  // fold back into literals, so each dequantised pair is one v_and_or_b32
  // (an instruction takes at most one literal) instead of an AND and an OR.
  uint32_t kNib, kBias;
  asm volatile("s_mov_b32 %0, 0xf000f" : "=s"(kNib));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(kBias));

  auto compute = [&](int ks, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    // dequantised weights: 128 + q as bf16, pairs (k, k+4) of each 8-k run
    v4i wd[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t w = (uint32_t)wq[slot][cb][d];
#pragma unroll
        for (int i = 0; i < 4; ++i) wd[cb][d][i] = (int)(((w >> (4 * i)) & kNib) | kBias);
      }
    float sf[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) sf[cb] = (float)__builtin_bit_cast(_Float16, sm.sc[ks & (C::kScG - 1)][scol[cb]]);
    const uint8_t* ab = &sm.a[ks & 1][0];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      v4i x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = *(const v4i*)(ab + aoff_rd[i] + rb * 4096);
      v4i af[4];  // per MFMA d: (a0,a4) (a1,a5) (a2,a6) (a3,a7) of the 8-k run
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t i0 = (uint32_t)x[d][0], i1 = (uint32_t)x[d][1], i2 = (uint32_t)x[d][2], i3 = (uint32_t)x[d][3];
        af[d] = v4i{(int)__builtin_amdgcn_perm(i2, i0, 0x05040100u), (int)__builtin_amdgcn_perm(i2, i0, 0x07060302u),
                    (int)__builtin_amdgcn_perm(i3, i1, 0x05040100u), (int)__builtin_amdgcn_perm(i3, i1, 0x07060302u)};
      }
      v4f corr = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < 4; ++d) corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(af[d]), as_bf(kNeg136), corr, 0, 0, 0);
      // four independent accumulation chains, interleaved so that no matrix
      // instruction waits on the one issued just before it
      v4f p[4];
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          p[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(af[d]), as_bf(wd[cb][d]), d == 0 ? corr : p[cb], 0, 0, 0);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[rb][cb][v] = __builtin_fmaf(sf[cb], p[cb][v], acc[rb][cb][v]);
    }
  };

  auto step = [&](int ks, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    commit(ks, s_c);
    barrier_lds();
    if (C::kScG < kMaxKBlocks && ks > 0 && (ks & (C::kScG - 1)) == 0) {
      stage_scales(ks);  // every wave is past the previous group's reads
      barrier_lds();
    }
    issue(ks + S - 1, IntC<(s + S - 1) % S>{});
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this block's MFMAs
    compute(ks, s_c);
  };

  static_for<0, S - 1>([&](auto s_c) { issue(decltype(s_c)::value, s_c); });
  const int nfull = KG / S;
  for (int g = 0; g < nfull; ++g) static_for<0, S>([&](auto s_c) { step(g * S + decltype(s_c)::value, s_c); });
  static_for<0, S>([&](auto s_c) {
    const int ks = nfull * S + decltype(s_c)::value;
    if (ks < KG) step(ks, s_c);
  });
  barrier_lds();

  if (wave_on) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 16 * rb + 4 * lg + v;
        if (m < u.mrows) {
          uint16_t* drow = a.D + (int64_t)(u.row0 + m) * N + ncol0 + l16;
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) drow[16 * cb] = (uint16_t)f32_to_bf16_rne(acc[rb][cb][v]);
        }
      }
  }
}

template <int RB, int S>
__global__ __launch_bounds__(256, 1) void gemm_int4_kernel(const GemmArgs a) {
  using C = I4Cfg<RB, S>;
  __shared__ __attribute__((aligned(1024))) I4Smem<RB, S> sm;
  __shared__ SchedSmem s_sched;
  const Sched sc{&s_sched};
  sched_build<C::BM>(a, sc);
  const Walk walk = sched_walk(s_sched.total);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const Unit u = sched_unit<C::BM>(a, sc, v);
    int4_unit<RB, S>(a, u, sm, wv, lane);
  }
}

// ------------------------------------------------------- packed weights --
template <int S, int SA>
__device__ __forceinline__ void int4_unit_packed(const GemmArgs& a, const Unit& u, int sub, int lane) {
  static_assert(S % SA == 0, "the activation ring must divide the weight ring");
  const int l16 = lane & 15, lg = lane >> 4;
  const int K = a.K, N = a.N, KG = K / 128;
  const int ncol0 = u.n0 + 64 * sub;
  if (ncol0 >= N) return;  // N is a multiple of 128: a wave with work has 64 whole columns

  // weights: group g of 16-column block b is 1 KB at (g*(N/16) + b)*1024; lane L's 16 bytes at 16L
  const uint8_t* wbase = a.W + (int64_t)u.e * N * (K / 2) + (int64_t)(ncol0 / 16) * 1024 + 16 * lane;
  const uint32_t wstep = (uint32_t)N * 64u;
  // scales [K/128][N/64][16][4]: the 4 column blocks of column l16 of this wave's 64, per group
  const uint16_t* sbase = (const uint16_t*)a.SW + (int64_t)u.e * N * KG + ncol0 + 4 * l16;
  // activations: row l16 (clamped to the unit's rows), 16 bytes per matrix instruction d at
  // k = 128g + 8(4d + lg): byte 256g + 64d + 16lg of the row
  const uint8_t* abase = a.A + ((int64_t)u.row0 + min(l16, u.mrows - 1)) * K * 2 + 16 * lg;

  v4i wq[S][4];
  uint2 sq[S];
  v4i ar[SA][4];
  v4f acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = v4f{0.f, 0.f, 0.f, 0.f};

  auto issue_w = [&](int ks_req, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const uint32_t ks = (uint32_t)min(ks_req, KG - 1);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)  // read once: streamed past the caches
      wq[slot][cb] = __builtin_nontemporal_load((const v4i*)(wbase + (ks * wstep + 1024u * cb)));
    sq[slot] = *(const uint2*)(sbase + ks * (uint32_t)N);
  };
  auto issue_a = [&](int ks_req, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const uint32_t ks = (uint32_t)min(ks_req, KG - 1);
#pragma unroll
    for (int d = 0; d < 4; ++d) ar[slot][d] = *(const v4i*)(abase + (ks * 256u + 64u * d));
  };

  const v4i kNeg136 = v4i{(int)0xC308C308u, (int)0xC308C308u, (int)0xC308C308u, (int)0xC308C308u};
  uint32_t kNib, kBias;  // registers, not literals: one v_and_or_b32 per dequantised pair
  asm volatile("s_mov_b32 %0, 0xf000f" : "=s"(kNib));
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(kBias));

  auto compute = [&](auto s_c) {
    constexpr int s = decltype(s_c)::value, sa = s % SA;
    const uint32_t s01 = sq[s].x, s23 = sq[s].y;
    const float sf[4] = {(float)__builtin_bit_cast(_Float16, (uint16_t)(s01 & 0xffffu)),
                         (float)__builtin_bit_cast(_Float16, (uint16_t)(s01 >> 16)),
                         (float)__builtin_bit_cast(_Float16, (uint16_t)(s23 & 0xffffu)),
                         (float)__builtin_bit_cast(_Float16, (uint16_t)(s23 >> 16))};
    v4f corr = v4f{0.f, 0.f, 0.f, 0.f};  // -136 * sum of the group's activations, per row
#pragma unroll
    for (int d = 0; d < 4; ++d) corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(ar[sa][d]), as_bf(kNeg136), corr, 0, 0, 0);
    v4f p[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const uint32_t w = (uint32_t)wq[s][cb][d];
        v4i wd;
#pragma unroll
        for (int i = 0; i < 4; ++i) wd[i] = (int)(((w >> (4 * i)) & kNib) | kBias);  // 128 + q, bf16 pairs
        p[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(ar[sa][d]), as_bf(wd), d == 0 ? corr : p[cb], 0, 0, 0);
      }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[cb][v] = __builtin_fmaf(sf[cb], p[cb][v], acc[cb][v]);
  };

  auto step = [&](int ks, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    issue_w(ks + S - 1, IntC<(s + S - 1) % S>{});
    issue_a(ks + SA - 1, IntC<(s + SA - 1) % SA>{});
    compute(s_c);
  };

  static_for<0, S - 1>([&](auto s_c) { issue_w(decltype(s_c)::value, s_c); });
  static_for<0, SA - 1>([&](auto s_c) { issue_a(decltype(s_c)::value, s_c); });
  const int nfull = KG / S;
  for (int g = 0; g < nfull; ++g) static_for<0, S>([&](auto s_c) { step(g * S + decltype(s_c)::value, s_c); });
  static_for<0, S>([&](auto s_c) {
    const int ks = nfull * S + decltype(s_c)::value;
    if (ks < KG) step(ks, s_c);
  });

#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * lg + v;
    if (m < u.mrows) {
      uint16_t* drow = a.D + (int64_t)(u.row0 + m) * N + ncol0 + l16;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) drow[16 * cb] = (uint16_t)f32_to_bf16_rne(acc[cb][v]);
    }
  }
}

// Ring depths (K groups in flight per wave) and workgroups per CU of the
// packed kernel.
#ifndef MOE_I4P_S
#define MOE_I4P_S 2
#endif
#ifndef MOE_I4P_SA
#define MOE_I4P_SA 2
#endif
#ifndef MOE_I4P_WGPC
#define MOE_I4P_WGPC 2
#endif

// The waves of a workgroup share nothing, so the work is dealt per wave: a
// wave's unit is 64 columns of a 256-column unit of the table (its sub-tile
// sub = v % 4), and the units go round-robin over all waves of the grid, wave
// slot wv * G + blockIdx.x first, so consecutive units (the column tiles of
// one expert, of equal cost) land on different workgroups and CUs.
template <int S, int SA, int WGPC>
__global__ __launch_bounds__(256, WGPC) void gemm_int4_packed_kernel(const GemmArgs a) {
  __shared__ SchedSmem s_sched;
  const Sched sc{&s_sched};
  sched_build<16>(a, sc);
  const int total = uniform(s_sched.total) * 4;
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  const int G = gridDim.x;
  for (int v = wv * G + blockIdx.x; v < total; v += 4 * G) {
    const Unit u = sched_unit<16>(a, sc, v >> 2);
    int4_unit_packed<S, SA>(a, u, v & 3, lane);
  }
}

template <int RB, int S>
static hipError_t launch_i4(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  gemm_int4_kernel<RB, S><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int S, int SA, int WGPC>
static hipError_t launch_i4p(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  gemm_int4_packed_kernel<S, SA, WGPC><<<WGPC * grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_int4(const GemmArgs& a, int expected_m, hipStream_t s) {
  if (a.wpacked) return launch_i4p<MOE_I4P_S, MOE_I4P_SA, MOE_I4P_WGPC>(a, s);  // 16-row units whatever the rows
  const int em = expected_m > 0 ? expected_m : (a.masked ? a.max_m : 64);
  if (em <= 16) return launch_i4<1, 8>(a, s);
  return launch_i4<4, 4>(a, s);
}

}  // namespace moe
