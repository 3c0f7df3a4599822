// gemm_int8.hip -- INT8 (1, 1, 128) grouped GEMM for gfx950.
//
// D[p, n] = bf16( sum_kb sa[p,kb] * sw[e,kb,n] * sum_{k in kb} a[p,k] * w[e,n,k] )
// (AsymGEMM README, "API Reference", INT8 asymmetric GEMM: int8 data with fp32
// scales of fixed granularity (1, 1, 128), one per token row and 128 K for the
// activations and one per output channel and 128 K for the weights, contiguous
// and masked layouts, bf16 output; the README's facade hands the weight scales
// to the kernel transposed, and this kernel takes them K-block-major,
// [E, K/128, N], as moe_quant_weight_int8 writes them.)
//
// Design for CDNA4:
//  * Matrix core: v_mfma_i32_16x16x64_i8, two per 128-wide K block, summed
//    exactly in int32 (|sum| <= 127 * 127 * 128 < 2^24, so its fp32 value is
//    exact too).  The block's sum is then promoted into the fp32 accumulator:
//    acc += float(sum) * (sa * sw).  The scales are per row and per column,
//    so unlike the FP8 path (one power-of-two scale per 128 columns, applied by
//    the scaled matrix instruction) the promotion is VALU work: three
//    operations per accumulator element and K block against two matrix
//    instructions per 16x16 tile, which bounds a compute-bound tile at about
//    2/3 of the int8 matrix peak.
//  * Tiles, rings and scheduling follow the short FP8 tiles: the weight tile
//    is the instruction's A operand (16 output columns), the activations its B
//    operand (16 rows); each wave owns 256/NW columns and streams their weight
//    fragments and weight scales from HBM into an S-deep register ring; the
//    activation row slices and their scales go through registers into two
//    XOR-swizzled LDS slots shared by the waves.  A lane's weight scales for
//    a K block are 4 consecutive columns of the K-block-major scale rows: one
//    16-byte load per 16-column block.
//  * Decode-sized segments: 16-row units, 4 waves of 64 columns, 3-deep ring.
//    Larger segments: 192-row units (a DeepSeek-V3-shaped prefill expert of
//    about 128 rows is one unit, so its weights stream once), 8 waves of 32
//    columns (two per SIMD, so one wave's promotion overlaps the other's
//    matrix instructions), 2-deep ring; the computed height is the smallest
//    of 64, 96, 128, 160 and 192 rows that covers the unit.  Within a K
//    block, row block rb's matrix instructions are issued before row block
//    rb - 1 is promoted.  Measured on the DeepSeek-V3-shaped prefill (32768
//    routed rows, N 4096, K 7168): 64-row units with 4 waves 3.5 ms, 128-row
//    units with 8 waves 2.6 ms, 192-row units 2.2 ms, 2.07 ms with the 96-
//    and 160-row heights; deeper rings, weight scales staged through LDS,
//    and a 2 x 4 wave layout that halves the LDS fragment reads were not
//    faster.
//  * The K-to-lane assignment of the two instructions is the same for both
//    operands (lane group g supplies bytes 16g..16g+15 of the block to the
//    first and 64+16g.. to the second), so the row-major weights and the
//    fragment order of moe_pack_weight_fp8 (a byte permutation, valid for any
//    one-byte code) both work.
//  * Scheduler: gemm_common.h (persistent, atomic-free, XCD-sliced).
#include "gemm_common.h"

namespace moe {

#ifndef MOE_I8_RB
#define MOE_I8_RB 12
#define MOE_I8_S 2
#define MOE_I8_NW 8
#endif

// RB: 16-row blocks per unit (BM = 16*RB); S: register-ring depth (K blocks);
// NW: waves per workgroup, each owning CB = 16/NW blocks of 16 columns (BN = 256).
template <int RB, int S, int NW>
struct Int8Cfg {
  static constexpr int BM = 16 * RB;
  static constexpr int CB = 16 / NW;
  static constexpr int kWcols = 16 * CB;               // columns per wave
  static constexpr int kApw = (2 * RB + NW - 1) / NW;  // 16-byte A loads per lane per stage (1 KB = 8 rows each)
  static constexpr int kArows = NW * 8 * kApw;         // rows held per LDS slot (>= BM)
  static constexpr int kAStage = kArows * 128;         // bytes per LDS slot
  static constexpr int kSaStage = NW * 64;             // row-scale floats per slot (one per lane)
  static_assert(kArows >= BM, "A stage too small");
  static_assert(S >= 2, "ring depth");
  static_assert(NW * CB == 16, "256 columns per unit");
};

template <int RB, int S, int NW>
struct Int8Smem {
  uint8_t a[2][Int8Cfg<RB, S, NW>::kAStage];
  float sa[2][Int8Cfg<RB, S, NW>::kSaStage];
};

// One unit with RBE (<= RB) row blocks computed.
template <int RB, int S, int NW, int RBE>
__device__ __forceinline__ void int8_unit(const GemmArgs& a, const Unit& u, Int8Smem<RB, S, NW>& sm, int wv,
                                          int lane) {
  using C = Int8Cfg<RB, S, NW>;
  constexpr int CB = C::CB;
  const int l16 = lane & 15, lg = lane >> 4;
  const int K = a.K, N = a.N, KB = K / 128;
  const int ncol0 = u.n0 + C::kWcols * wv;  // this wave's first column
  const bool wave_on = ncol0 < N;

  // weight bytes: uniform expert base + 32-bit lane offset (columns clamped for an idle wave); the layouts as
  // in the FP8 short tiles
  const uint8_t* wbase = a.W + (int64_t)u.e * N * K;
  const uint32_t wstep = a.wpacked ? (uint32_t)N * 128u : 128u;  // bytes per K block
  const uint32_t whalf = a.wpacked ? 1024u : 64u;
  uint32_t woff[CB];
  uint32_t soff[CB];  // this lane's 4 weight-scale columns within a K block's scale row
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    int n = ncol0 + 16 * cb + l16;
    if (n >= N) n = N - 1;
    woff[cb] = a.wpacked ? (uint32_t)(n / 16) * 2048u + 16u * lane : (uint32_t)n * (uint32_t)K + 16u * lg;
    int ns = ncol0 + 16 * cb + 4 * lg;
    if (ns > N - 4) ns = N - 4;
    soff[cb] = (uint32_t)ns;
  }
  const float* swbase = (const float*)a.SW + (int64_t)u.e * KB * N;
  // activation rows this lane's loads fetch (clamped to valid rows)
  const uint8_t* abase = a.A + (int64_t)u.row0 * K;
  uint32_t aoff[C::kApw];
#pragma unroll
  for (int i = 0; i < C::kApw; ++i) {
    const int q = wv * C::kApw + i;             // 1 KB block of the stage this lane writes into
    const int r = 8 * q + (lane >> 3);          // tile row written by this lane
    const int c = (lane & 7) ^ ((r >> 1) & 7);  // chunk that lands at position lane & 7
    aoff[i] = (uint32_t)min(r, u.mrows - 1) * (uint32_t)K + 16u * c;
  }
  const float* sarow = a.SFA + (int64_t)(u.row0 + min(64 * wv + lane, u.mrows - 1)) * KB;  // rows >= BM unused

  // fragment read offsets: row m = 16*rb + l16 at m*128, chunk c at position
  // c ^ ((m >> 1) & 7); that term does not depend on rb.
  const int fsw = (l16 >> 1) & 7;
  const int off_lo = l16 * 128 + 16 * (lg ^ fsw);
  const int off_hi = l16 * 128 + 16 * ((4 + lg) ^ fsw);

  v4i wlo[S][CB], whi[S][CB];
  v4f wsc[S][CB];
  v4i ar[S][C::kApw];
  float sr[S];
  v4f acc[RBE][CB];
#pragma unroll
  for (int rb = 0; rb < RBE; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int ks_req, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const int ks = min(ks_req, KB - 1);
    const uint32_t koff = (uint32_t)ks * 128u, wkoff = (uint32_t)ks * wstep;
    const float* swk = swbase + (int64_t)ks * N;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const v4i* wl = (const v4i*)(wbase + (woff[cb] + wkoff));
      const v4i* wh = (const v4i*)(wbase + (woff[cb] + wkoff + whalf));
      if constexpr (RB == 1) {
        // decode-sized units read each weight byte once: stream past the caches
        wlo[slot][cb] = __builtin_nontemporal_load(wl);
        whi[slot][cb] = __builtin_nontemporal_load(wh);
      } else {
        wlo[slot][cb] = *wl;
        whi[slot][cb] = *wh;
      }
      wsc[slot][cb] = *(const v4f*)(swk + soff[cb]);
    }
#pragma unroll
    for (int i = 0; i < C::kApw; ++i) ar[slot][i] = *(const v4i*)(abase + (aoff[i] + koff));
    sr[slot] = sarow[ks];
  };

  // stage registers -> LDS slot (ks & 1)
  auto commit = [&](int ks, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    uint8_t* dst = &sm.a[ks & 1][0];
#pragma unroll
    for (int i = 0; i < C::kApw; ++i) *(v4i*)(dst + (wv * C::kApw + i) * 1024 + 16 * lane) = ar[slot][i];
    sm.sa[ks & 1][64 * wv + lane] = sr[slot];
  };

  // Row block rb's matrix instructions are issued before row block rb - 1 is
  // promoted, and rb + 1's fragments are read meanwhile, so the VALU work of
  // one row block overlaps the matrix pipe and LDS latency of the next.
  auto compute = [&](int ks, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const uint8_t* ab = &sm.a[ks & 1][0];
    const float* sab = &sm.sa[ks & 1][l16];
    v4i alo[2], ahi[2], sum[2][CB];
    alo[0] = *(const v4i*)(ab + off_lo);
    ahi[0] = *(const v4i*)(ab + off_hi);
    auto promote = [&](int rb, int b) {
      const float sa = sab[16 * rb];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[rb][cb][r] = fmaf((float)sum[b][cb][r], sa * wsc[slot][cb][r], acc[rb][cb][r]);
    };
#pragma unroll
    for (int rb = 0; rb < RBE; ++rb) {
      const int b = rb & 1;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        sum[b][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo[slot][cb], alo[b], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        sum[b][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi[slot][cb], ahi[b], sum[b][cb], 0, 0, 0);
      if (rb + 1 < RBE) {
        alo[b ^ 1] = *(const v4i*)(ab + off_lo + (rb + 1) * 2048);
        ahi[b ^ 1] = *(const v4i*)(ab + off_hi + (rb + 1) * 2048);
      }
      if (rb > 0) promote(rb - 1, b ^ 1);
    }
    promote(RBE - 1, (RBE - 1) & 1);
  };

  // One K block: publish its activations, refill the ring, multiply.  LDS
  // slot ks&1 was last read two steps ago, before the previous barrier.
  auto step = [&](int ks, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    commit(ks, s_c);
    barrier_lds();
    issue(ks + S - 1, IntC<(s + S - 1) % S>{});
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this block's matrix instructions
    compute(ks, s_c);
  };

  static_for<0, S - 1>([&](auto s_c) { issue(decltype(s_c)::value, s_c); });
  const int nfull = KB / S;
  for (int g = 0; g < nfull; ++g) static_for<0, S>([&](auto s_c) { step(g * S + decltype(s_c)::value, s_c); });
  static_for<0, S>([&](auto s_c) {
    const int ks = nfull * S + decltype(s_c)::value;
    if (ks < KB) step(ks, s_c);
  });
  barrier_lds();  // every wave is done with both LDS slots before the next unit refills them

  if (wave_on) {
#pragma unroll
    for (int rb = 0; rb < RBE; ++rb) {
      const int m = 16 * rb + l16;
      if (m < u.mrows) {
        uint16_t* drow = a.D + (int64_t)(u.row0 + m) * N + ncol0 + 4 * lg;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          uint2 o;
          o.x = f32_to_bf16_rne(acc[rb][cb][0]) | (f32_to_bf16_rne(acc[rb][cb][1]) << 16);
          o.y = f32_to_bf16_rne(acc[rb][cb][2]) | (f32_to_bf16_rne(acc[rb][cb][3]) << 16);
          *(uint2*)(drow + 16 * cb) = o;
        }
      }
    }
  }
}

template <int RB, int S, int NW>
__global__ __launch_bounds__(NW * 64, 1) void gemm_int8_kernel(const GemmArgs a) {
  using C = Int8Cfg<RB, S, NW>;
  __shared__ __attribute__((aligned(1024))) Int8Smem<RB, S, NW> sm;
  __shared__ SchedSmem s_sched;

  const Sched sc{&s_sched};
  sched_build<C::BM>(a, sc);
  const Walk walk = sched_walk(s_sched.total);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const Unit u = sched_unit<C::BM>(a, sc, v);
    // computed height: the smallest of 64, 96, 128, 160, 192 rows (RB = 12) that covers the unit, or a half of
    // the full height; padding rows are never stored
    if constexpr (RB == 12) {
      if (u.mrows <= 64) int8_unit<RB, S, NW, 4>(a, u, sm, wv, lane);
      else if (u.mrows <= 96) int8_unit<RB, S, NW, 6>(a, u, sm, wv, lane);
      else if (u.mrows <= 128) int8_unit<RB, S, NW, 8>(a, u, sm, wv, lane);
      else if (u.mrows <= 160) int8_unit<RB, S, NW, 10>(a, u, sm, wv, lane);
      else int8_unit<RB, S, NW, 12>(a, u, sm, wv, lane);
    } else if constexpr (RB > 1) {
      if (u.mrows <= 16 * ((RB + 1) / 2)) int8_unit<RB, S, NW, (RB + 1) / 2>(a, u, sm, wv, lane);
      else int8_unit<RB, S, NW, RB>(a, u, sm, wv, lane);
    } else {
      int8_unit<RB, S, NW, 1>(a, u, sm, wv, lane);
    }
  }
}

template <int RB, int S, int NW>
static hipError_t launch_int8(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  gemm_int8_kernel<RB, S, NW><<<grid, NW * 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_int8(const GemmArgs& a, int expected_m, hipStream_t s) {
  // decode-sized segments: one 16-row block per unit, weights streamed once; larger ones: 64-row units
  const int em = expected_m > 0 ? expected_m : (a.masked ? a.max_m : 256);
  if (em <= 16) return launch_int8<1, 3, 4>(a, s);
  return launch_int8<MOE_I8_RB, MOE_I8_S, MOE_I8_NW>(a, s);
}

}  // namespace moe
