// gemm_fp8.hip -- block-scaled FP8 grouped GEMM for gfx950.
//
// D[p, n] = bf16( sum_kb sa[p,kb] * sw[e,n/128,kb] * sum_{k in kb} a[p,k] * w[e,n,k] )
// (rainlin, "GEMM 执行方式", sec. 4.4: Y_e = X_e W_e^T per expert; AsymGEMM
// README "API Reference": FP8 (data, scale) operands with 1x128 activation and
// 128x128 weight scales, contiguous and masked layouts, bf16 output;
// nxmr.cn DeepGEMM article: FP32 accumulation, power-of-two block scales.)
//
// Design for CDNA4:
//  * Matrix core: v_mfma_scale_f32_16x16x128_f8f6f4.  One instruction covers
//    exactly one 128-wide K block and applies an E8M0 scale per row of each
//    operand; the pow2 fp32 scales ARE E8M0 (their biased exponent), so the
//    per-block scale promotion into the FP32 accumulator costs no VALU work and
//    is exact.  The weight tile is the instruction's A operand (16 output
//    columns n), the activations its B operand (16 rows m): the accumulator
//    layout then gives each lane 4 consecutive n of one row (one 8-byte store).
//  * Weights: each wave owns 64 columns for the whole unit; its weight
//    fragments stream from HBM straight into VGPRs through an S-deep register
//    ring (S-1 K blocks in flight per wave), no LDS round trip.
//  * Activations: shared by the 4 waves.  Each stage's 128-byte row slices
//    are loaded into VGPRs with the weights (same ring depth), then written
//    to one of two LDS slots XOR-swizzled so fragment reads are bank-conflict
//    free; the row scales ride along.  All loads are plain vector loads, so the
//    compiler's wait counts stay exact.  Each wave's weight scales for the unit
//    are staged once per unit.
//  * Every stage issues the same loads (the tail re-reads the last K block
//    instead of skipping), so the wait pattern is identical for every stage.
//  * Rows: a unit holds at most BM = 16*RB rows; it runs with the smaller of
//    two tile heights that covers its valid rows, and padding rows are never
//    stored.
//  * Scheduler: gemm_common.h (persistent, atomic-free, XCD-sliced).
#include "gemm_common.h"

namespace moe {

// RB: 16-row blocks per unit (BM = 16*RB); S: register-ring depth (K blocks);
// NW: waves per workgroup, each owning CB = 16/NW blocks of 16 columns (BN = 256).
template <int RB, int S, int NW>
struct Fp8Cfg {
  static constexpr int BM = 16 * RB;
  static constexpr int CB = 16 / NW;
  static constexpr int kWcols = 16 * CB;                  // columns per wave
  static constexpr int kApw = (2 * RB + NW - 1) / NW;     // 16-byte A loads per lane per stage (1 KB = 8 rows each)
  static constexpr int kArows = NW * 8 * kApw;            // rows held per LDS slot (>= BM)
  static constexpr int kAStage = kArows * 128;            // bytes per LDS slot
  static constexpr int kSaStage = NW * 64;                // scale floats per slot (one per lane)
  static_assert(kArows >= BM, "A stage too small");
  static_assert(S >= 2, "ring depth");
  static_assert(NW * CB == 16, "256 columns per unit");
};

template <int RB, int S, int NW>
struct Fp8Smem {
  uint8_t a[2][Fp8Cfg<RB, S, NW>::kAStage];
  float sa[2][Fp8Cfg<RB, S, NW>::kSaStage];
  float sw[NW][kMaxKBlocks];  // per-wave weight scales of the current unit
};

// One unit with RBE (<= RB) row blocks computed.
template <int RB, int S, int NW, int RBE>
__device__ __forceinline__ void fp8_unit(const GemmArgs& a, const Unit& u, Fp8Smem<RB, S, NW>& sm, int wv,
                                         int lane) {
  using C = Fp8Cfg<RB, S, NW>;
  constexpr int CB = C::CB;
  const int l16 = lane & 15, lg = lane >> 4;
  const int K = a.K, N = a.N, KB = K / 128, NB = N / 128;
  const int ncol0 = u.n0 + C::kWcols * wv;  // this wave's first column
  const bool wave_on = ncol0 < N;

  // weight bytes: uniform expert base + 32-bit lane offset (rows clamped for an idle wave)
  const uint8_t* wbase = a.W + (int64_t)u.e * N * K;
  uint32_t woff[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    int n = ncol0 + 16 * cb + l16;
    if (n >= N) n = N - 1;
    woff[cb] = (uint32_t)n * (uint32_t)K + 16u * lg;
  }
  // this wave's 128-column block of weight scales for the whole unit -> LDS
  const float* sw_ptr = (const float*)a.SW + ((int64_t)u.e * NB + (wave_on ? ncol0 : 0) / 128) * KB;
  for (int j = 0; j < KB; j += 64) sm.sw[wv][j + lane] = sw_ptr[min(j + lane, KB - 1)];
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

  v8i wf[S][CB];
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
    const uint32_t koff = (uint32_t)ks * 128u;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const v4i lo = *(const v4i*)(wbase + (woff[cb] + koff));
      const v4i hi = *(const v4i*)(wbase + (woff[cb] + koff + 64u));
      wf[slot][cb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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

  auto compute = [&](int ks, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const int swe = (int)(__float_as_uint(sm.sw[wv][ks]) >> 23);
    const uint8_t* ab = &sm.a[ks & 1][0];
    const float* sab = &sm.sa[ks & 1][l16];
#pragma unroll
    for (int rb = 0; rb < RBE; ++rb) {
      const v4i lo = *(const v4i*)(ab + off_lo + rb * 2048);
      const v4i hi = *(const v4i*)(ab + off_hi + rb * 2048);
      const v8i af = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int sae = (int)(__float_as_uint(sab[16 * rb]) >> 23);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[slot][cb], af, acc[rb][cb], 0, 0, 0, swe,
                                                                       0, sae);
    }
  };

  // One K block: publish its activations, refill the ring, multiply.  LDS
  // slot ks&1 was last read two steps ago, before the previous barrier.
  auto step = [&](int ks, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    commit(ks, s_c);
    barrier_lds();
    issue(ks + S - 1, IntC<(s + S - 1) % S>{});
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this block's MFMAs
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
__global__ __launch_bounds__(NW * 64, 1) void gemm_fp8_kernel(const GemmArgs a) {
  using C = Fp8Cfg<RB, S, NW>;
  __shared__ __attribute__((aligned(1024))) Fp8Smem<RB, S, NW> sm;
  __shared__ int s_up[kMaxExperts + 1], s_tmp[NW * 64 + 1];

  const Sched sc{s_up};
  sched_build<C::BM>(a, sc, s_tmp);
  const Walk walk = sched_walk(s_up[a.E]);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  constexpr int RH = (RB + 1) / 2;  // the shorter tile height

  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const Unit u = sched_unit<C::BM>(a, sc, v);
    if (RB > 1 && u.mrows <= 16 * RH) fp8_unit<RB, S, NW, RH>(a, u, sm, wv, lane);
    else fp8_unit<RB, S, NW, RB>(a, u, sm, wv, lane);
  }
}

// ----------------------------------------------------------------------------
// Tall tiles (prefill): BM = 192 rows x BN = 256 columns, 4 waves of 64
// columns, K consumed in halves of 64 bytes with v_mfma_scale_f32_32x32x64_f8f6f4
// (the two halves of a 128-wide K block share its scales).  Both operands are
// staged in LDS by direct global->LDS copies in a 5-deep ring (4 half-blocks,
// ~112 KB per CU, in flight while one is multiplied).  Each wave's weight slab
// (64 rows x 64 B per half block) is private to it; the activation tile is
// shared.  The copies are inline asm (moe_device.h), so the waits on them are
// explicit: a wave issues kLOps copies per stage, and "stage h landed" is
// vmcnt <= kLOps * (stages issued after h).  Registers hold the accumulators
// and one row block's fragments only.
constexpr int kLRB = 6;                    // 32-row blocks (BM = 192)
constexpr int kLS = 5;                     // LDS ring depth (half blocks)
constexpr int kLWslab = 64 * 64;           // one wave's weight slab per stage (bytes)
constexpr int kLAtile = 32 * kLRB * 64;    // activation tile per stage (bytes)
constexpr int kLApw = kLAtile / 1024 / 4;  // activation copies per wave per stage
constexpr int kLOps = 4 + kLApw + 1;       // copies per wave per stage (weights, activations, row scales)

struct Fp8LdsSmem {
  uint8_t w[kLS][4][kLWslab];
  uint8_t a[kLS][kLAtile];
  float sa[kLS][256];
  float sw[4][kMaxKBlocks];  // per-wave weight scales of the current unit
};

typedef float v16f __attribute__((ext_vector_type(16)));
// An empty asm that reads and writes x in AGPRs: fixes where x is produced.
__device__ __forceinline__ void pin_agpr(v16f& x) { asm volatile("" : "+a"(x)); }

template <int N>
__device__ __forceinline__ void wait_vmcnt_rt(int n) {  // n in [0, N], multiples of kLOps
  if (n >= 3 * kLOps) wait_vmcnt<3 * kLOps>();
  else if (n >= 2 * kLOps) wait_vmcnt<2 * kLOps>();
  else if (n >= kLOps) wait_vmcnt<kLOps>();
  else wait_vmcnt<0>();
}

// 64-byte rows: the 16-byte chunk c of row r sits at position c ^ ((r >> 2) & 3).
template <int RBE>
__device__ __forceinline__ void fp8_unit_lds(const GemmArgs& a, const Unit& u, Fp8LdsSmem& sm, int wv, int lane) {
  const int l32 = lane & 31, lh = lane >> 5;
  const int K = a.K, N = a.N, KB = K / 128, KH = K / 64, NB = N / 128;
  const int ncol0 = u.n0 + 64 * wv;
  const bool wave_on = ncol0 < N;
  const int ncl = wave_on ? ncol0 : N - 64;  // an idle wave re-reads valid rows and stores nothing

  // copy sources (16 rows of 64 B per copy instruction)
  const uint8_t* wsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * i + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    wsrc[i] = a.W + ((int64_t)u.e * N + ncl + r) * K + 16 * c;
  }
  const uint8_t* asrc[kLApw];
#pragma unroll
  for (int i = 0; i < kLApw; ++i) {
    const int r = 16 * (wv * kLApw + i) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    asrc[i] = a.A + (int64_t)(u.row0 + min(r, u.mrows - 1)) * K + 16 * c;
  }
  const float* sasrc = a.SFA + (int64_t)(u.row0 + min(64 * wv + lane, u.mrows - 1)) * KB;
  // this wave's weight scales for the unit -> LDS, with ordinary loads before any copy is in flight
  const float* swsrc = (const float*)a.SW + ((int64_t)u.e * NB + ncl / 128) * KB;
  for (int j = 0; j < KB; j += 64) sm.sw[wv][j + lane] = swsrc[min(j + lane, KB - 1)];

  // fragment reads: lane (row r = l32, half lh) takes chunks lh and 2 + lh of its row
  const int fsw = (l32 >> 2) & 3;
  const int off_lo = l32 * 64 + 16 * (lh ^ fsw);
  const int off_hi = l32 * 64 + 16 * ((2 + lh) ^ fsw);

  v16f acc[RBE][2];
#pragma unroll
  for (int rb = 0; rb < RBE; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.f;

  auto issue = [&](int h, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const int koff = h * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(wsrc[i] + koff, &sm.w[slot][wv][i * 1024]);
#pragma unroll
    for (int i = 0; i < kLApw; ++i) dma16(asrc[i] + koff, &sm.a[slot][(wv * kLApw + i) * 1024]);
    dma4(sasrc + (h >> 1), &sm.sa[slot][64 * wv]);
  };

  auto compute = [&](int h, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const int swe = (int)(__float_as_uint(sm.sw[wv][h >> 1]) >> 23);
    v8i wf[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const v4i lo = *(const v4i*)(&sm.w[slot][wv][0] + off_lo + cb * 2048);
      const v4i hi = *(const v4i*)(&sm.w[slot][wv][0] + off_hi + cb * 2048);
      wf[cb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    const uint8_t* ab = &sm.a[slot][0];
    const float* sab = &sm.sa[slot][l32];
#pragma unroll
    for (int rb = 0; rb < RBE; ++rb) {
      const v4i lo = *(const v4i*)(ab + off_lo + rb * 2048);
      const v4i hi = *(const v4i*)(ab + off_hi + rb * 2048);
      const v8i af = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int sae = (int)(__float_as_uint(sab[32 * rb]) >> 23);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[cb], af, acc[rb][cb], 0, 0, 0, swe, 0,
                                                                      sae);
    }
  };

  // Half block h is in slot h % 5.  Before multiplying it: its copies have
  // landed (the later stages already issued may stay in flight) and every wave
  // has passed the barrier, so slot (h + 4) % 5 -- last read for h - 1 -- is free.
  auto step = [&](int h, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    __builtin_amdgcn_sched_barrier(0);
    const int later = min(KH - 1 - h, kLS - 2);  // stages issued after h
    wait_vmcnt_rt<3 * kLOps>(later * kLOps);
    barrier_lds();
    if (h + kLS - 1 < KH) issue(h + kLS - 1, IntC<(s + kLS - 1) % kLS>{});
    __builtin_amdgcn_sched_barrier(0);
    compute(h, s_c);
    // Pin this half block's MFMAs here: without a use, the optimiser sinks the
    // pure MFMA chains to the end of the unrolled loop and keeps every stage's
    // fragments live at once.
#pragma unroll
    for (int rb = 0; rb < RBE; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) pin_agpr(acc[rb][cb]);
  };

  static_for<0, kLS - 1>([&](auto s_c) {
    constexpr int s = decltype(s_c)::value;
    if (s < KH) issue(s, s_c);
  });
  const int nfull = KH / kLS;
  for (int g = 0; g < nfull; ++g) static_for<0, kLS>([&](auto s_c) { step(g * kLS + decltype(s_c)::value, s_c); });
  static_for<0, kLS>([&](auto s_c) {
    const int h = nfull * kLS + decltype(s_c)::value;
    if (h < KH) step(h, s_c);
  });
  wait_vmcnt<0>();
  barrier_lds();  // the ring is free for the next unit

  // accumulator (32x32): lane holds column m = l32 and rows n = 8q + 4lh + j
  if (wave_on) {
#pragma unroll
    for (int rb = 0; rb < RBE; ++rb) {
      const int m = 32 * rb + l32;
      if (m < u.mrows) {
        uint16_t* drow = a.D + (int64_t)(u.row0 + m) * N + ncol0 + 4 * lh;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint2 o;
            o.x = f32_to_bf16_rne(acc[rb][cb][4 * q]) | (f32_to_bf16_rne(acc[rb][cb][4 * q + 1]) << 16);
            o.y = f32_to_bf16_rne(acc[rb][cb][4 * q + 2]) | (f32_to_bf16_rne(acc[rb][cb][4 * q + 3]) << 16);
            *(uint2*)(drow + 32 * cb + 8 * q) = o;
          }
      }
    }
  }
}

__global__ __launch_bounds__(256, 1) void gemm_fp8_lds_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) Fp8LdsSmem sm;
  __shared__ int s_up[kMaxExperts + 1];
  const Sched sc{s_up};
  // the scan scratch (257 ints) borrows the row-scale ring, which is idle until the first unit
  sched_build<32 * kLRB>(a, sc, (int*)&sm.sa[0][0]);
  const Walk walk = sched_walk(s_up[a.E]);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const Unit u = sched_unit<32 * kLRB>(a, sc, v);
    if (u.mrows <= 96) fp8_unit_lds<3>(a, u, sm, wv, lane);
    else fp8_unit_lds<kLRB>(a, u, sm, wv, lane);
  }
}

template <int RB, int S, int NW>
static hipError_t launch_fp8(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  gemm_fp8_kernel<RB, S, NW><<<grid, NW * 64, 0, s>>>(a);
  return hipGetLastError();
}

static hipError_t launch_fp8_lds(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  gemm_fp8_lds_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const GemmArgs& a, int expected_m, hipStream_t s) {
  // Tile height from the expected rows per active expert: decode-sized
  // segments keep the weights in a deep register ring (short tiles), prefill
  // segments use the LDS-staged 128-row tile.
  const int em = expected_m > 0 ? expected_m : (a.masked ? a.max_m : 256);
  if (em <= 16) return launch_fp8<1, 8, 4>(a, s);
  if (em <= 64) return launch_fp8<4, 6, 4>(a, s);
  return launch_fp8_lds(a, s);
}

}  // namespace moe
