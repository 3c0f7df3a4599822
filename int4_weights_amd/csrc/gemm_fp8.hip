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

template <int RB, int S>
struct Fp8Cfg {
  static constexpr int BM = 16 * RB;
  static constexpr int kApw = RB >= 2 ? RB / 2 : 1;       // 16-byte A loads per lane per stage
  static constexpr int kArows = 4 * 8 * kApw;             // rows held per stage (>= BM)
  static constexpr int kAStage = kArows * 128;            // bytes per LDS slot
  static constexpr int kSaStage = 256;                    // scale floats per slot (4 waves x 64)
  static_assert(kArows >= BM, "A stage too small");
  static_assert(S >= 2, "ring depth");
};

template <int RB, int S>
struct Fp8Smem {
  uint8_t a[2][Fp8Cfg<RB, S>::kAStage];
  float sa[2][Fp8Cfg<RB, S>::kSaStage];
  float sw[4][kMaxKBlocks];  // per-wave weight scales of the current unit
};

// One unit with RBE (<= RB) row blocks computed.
template <int RB, int S, int RBE>
__device__ __forceinline__ void fp8_unit(const GemmArgs& a, const Unit& u, Fp8Smem<RB, S>& sm, int wv, int lane) {
  using C = Fp8Cfg<RB, S>;
  const int l16 = lane & 15, lg = lane >> 4;
  const int K = a.K, N = a.N, KB = K / 128, NB = N / 128;
  const int ncol0 = u.n0 + 64 * wv;  // this wave's first column
  const bool wave_on = ncol0 < N;

  // weight bytes: uniform expert base + 32-bit lane offset (rows clamped for an idle wave)
  const uint8_t* wbase = a.W + (int64_t)u.e * N * K;
  uint32_t woff[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
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
  const float* sarow = a.SFA + (int64_t)(u.row0 + min(64 * wv + lane, u.mrows - 1)) * KB;

  // fragment read offsets: row m = 16*rb + l16 at m*128, chunk c at position
  // c ^ ((m >> 1) & 7); that term does not depend on rb.
  const int fsw = (l16 >> 1) & 7;
  const int off_lo = l16 * 128 + 16 * (lg ^ fsw);
  const int off_hi = l16 * 128 + 16 * ((4 + lg) ^ fsw);

  v8i wf[S][4];
  v4i ar[S][C::kApw];
  float sr[S];
  v4f acc[RBE][4];
#pragma unroll
  for (int rb = 0; rb < RBE; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int ks_req, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const int ks = min(ks_req, KB - 1);
    const uint32_t koff = (uint32_t)ks * 128u;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
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
      for (int cb = 0; cb < 4; ++cb)
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
        for (int cb = 0; cb < 4; ++cb) {
          uint2 o;
          o.x = f32_to_bf16_rne(acc[rb][cb][0]) | (f32_to_bf16_rne(acc[rb][cb][1]) << 16);
          o.y = f32_to_bf16_rne(acc[rb][cb][2]) | (f32_to_bf16_rne(acc[rb][cb][3]) << 16);
          *(uint2*)(drow + 16 * cb) = o;
        }
      }
    }
  }
}

template <int RB, int S>
__global__ __launch_bounds__(256, 1) void gemm_fp8_kernel(const GemmArgs a) {
  using C = Fp8Cfg<RB, S>;
  __shared__ __attribute__((aligned(1024))) Fp8Smem<RB, S> sm;
  __shared__ int s_rows[kMaxExperts], s_start[kMaxExperts], s_up[kMaxExperts + 1], s_tmp[257];

  const Sched sc{s_rows, s_start, s_up};
  sched_build<C::BM>(a, sc, s_tmp);
  const Walk walk = sched_walk(s_up[a.E]);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  constexpr int RH = (RB + 1) / 2;  // the shorter tile height

  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const Unit u = sched_unit<C::BM>(a, sc, v);
    if (RB > 1 && u.mrows <= 16 * RH) fp8_unit<RB, S, RH>(a, u, sm, wv, lane);
    else fp8_unit<RB, S, RB>(a, u, sm, wv, lane);
  }
}

template <int RB, int S>
static hipError_t launch_fp8(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  gemm_fp8_kernel<RB, S><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const GemmArgs& a, int expected_m, hipStream_t s) {
  // Tile height from the expected rows per active expert: decode-sized
  // segments get a short tile (more weight stages in flight), prefill a tall one.
  const int em = expected_m > 0 ? expected_m : (a.masked ? a.max_m : 256);
  if (em <= 16) return launch_fp8<1, 8>(a, s);
  if (em <= 64) return launch_fp8<4, 6>(a, s);
  return launch_fp8<12, 4>(a, s);
}

}  // namespace moe
