// gemm_bf16.hip -- BF16 grouped GEMM for gfx950 (contiguous and masked layouts).
//
// D[p, n] = bf16( sum_k a[p,k] * w[e,n,k] ), fp32 accumulation
// (AsymGEMM README, "API Reference": BF16 m_grouped contiguous and masked
// grouped GEMMs, NT operands, bf16 output; rainlin, "GEMM 执行方式", sec. 4.6:
// the BF16 contiguous grouped GEMM called on the packed segments.)
//
// The same design as the FP8 short tiles (gemm_fp8.hip), on the bf16 matrix
// instruction and without scales:
//  * scheduler: gemm_common.h (persistent, atomic-free, cost-sorted, dealt
//    per XCD); a unit is (expert, 256 columns, up to BM = 16 RB rows);
//  * each of the 4 waves owns 64 columns; one step covers 64 K values, i.e.
//    128 bytes of every row (the bytes of one FP8 K block), multiplied by two
//    v_mfma_f32_16x16x32_bf16 per 16 x 16 output block;
//  * weights stream from HBM straight into an S-deep register ring (S - 1
//    steps in flight per wave); activations are loaded with the weights and
//    staged through two XOR-swizzled LDS slots shared by the 4 waves;
//  * both operands use the same assignment of K to lanes: lane (row l16, group
//    lg) supplies elements 8 lg .. 8 lg + 7 of the step to the first
//    instruction and 32 + 8 lg .. 32 + 8 lg + 7 to the second;
//  * bf16 output by round to nearest even; rows outside the segments are
//    never written.
#include "gemm_common.h"

namespace moe {

template <int RB, int S>
struct Bf16Cfg {
  static constexpr int BM = 16 * RB;
  static constexpr int kApw = (2 * RB + 3) / 4;  // 16-byte A loads per lane per stage (1 KB = 8 rows x 128 B)
  static constexpr int kArows = 4 * 8 * kApw;    // rows held per LDS slot (>= BM)
  static constexpr int kAStage = kArows * 128;   // bytes per LDS slot
  static_assert(kArows >= BM, "A stage too small");
  static_assert(S >= 2, "ring depth");
};

template <int RB, int S>
struct Bf16Smem {
  uint8_t a[2][Bf16Cfg<RB, S>::kAStage];
};

__device__ __forceinline__ v8bf bf_of(const v4i& x) { return __builtin_bit_cast(v8bf, x); }

// One unit with RBE (<= RB) row blocks computed.
template <int RB, int S, int RBE>
__device__ __forceinline__ void bf16_unit(const GemmArgs& a, const Unit& u, Bf16Smem<RB, S>& sm, int wv, int lane) {
  using C = Bf16Cfg<RB, S>;
  const int l16 = lane & 15, lg = lane >> 4;
  const int K = a.K, N = a.N, KS = K / 64;
  const uint32_t rowb = (uint32_t)K * 2u;  // bytes per row of A and of W
  const int ncol0 = u.n0 + 64 * wv;        // this wave's first column
  const bool wave_on = ncol0 < N;

  // weights: column n's step ks is 128 bytes at n*2K + 128 ks; the lane's halves at +16 lg and +64 + 16 lg
  const uint8_t* wbase = a.W + (int64_t)u.e * N * rowb;
  uint32_t woff[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    int n = ncol0 + 16 * cb + l16;
    if (n >= N) n = N - 1;  // an idle wave re-reads valid columns and stores nothing
    woff[cb] = (uint32_t)n * rowb + 16u * lg;
  }
  // activation rows this lane's loads fetch (clamped to valid rows)
  const uint8_t* abase = a.A + (int64_t)u.row0 * rowb;
  uint32_t aoff[C::kApw];
#pragma unroll
  for (int i = 0; i < C::kApw; ++i) {
    const int q = wv * C::kApw + i;             // 1 KB block of the stage this lane writes into
    const int r = 8 * q + (lane >> 3);          // tile row written by this lane
    const int c = (lane & 7) ^ ((r >> 1) & 7);  // chunk that lands at position lane & 7
    aoff[i] = (uint32_t)min(r, u.mrows - 1) * rowb + 16u * c;
  }
  // fragment read offsets: row m = 16 rb + l16 at m*128, chunk c at position c ^ ((m >> 1) & 7)
  const int fsw = (l16 >> 1) & 7;
  const int off_lo = l16 * 128 + 16 * (lg ^ fsw);
  const int off_hi = l16 * 128 + 16 * ((4 + lg) ^ fsw);

  v4i wlo[S][4], whi[S][4];
  v4i ar[S][C::kApw];
  v4f acc[RBE][4];
#pragma unroll
  for (int rb = 0; rb < RBE; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int ks_req, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const uint32_t koff = (uint32_t)min(ks_req, KS - 1) * 128u;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const uint8_t* wp = wbase + (woff[cb] + koff);
      if constexpr (RB == 1) {
        // decode-sized units: an expert's rows fit one unit, so each weight byte is read once
        wlo[slot][cb] = __builtin_nontemporal_load((const v4i*)wp);
        whi[slot][cb] = __builtin_nontemporal_load((const v4i*)(wp + 64));
      } else {
        wlo[slot][cb] = *(const v4i*)wp;
        whi[slot][cb] = *(const v4i*)(wp + 64);
      }
    }
#pragma unroll
    for (int i = 0; i < C::kApw; ++i) ar[slot][i] = *(const v4i*)(abase + (aoff[i] + koff));
  };

  auto commit = [&](int ks, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    uint8_t* dst = &sm.a[ks & 1][0];
#pragma unroll
    for (int i = 0; i < C::kApw; ++i) *(v4i*)(dst + (wv * C::kApw + i) * 1024 + 16 * lane) = ar[slot][i];
  };

  auto compute = [&](int ks, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const uint8_t* ab = &sm.a[ks & 1][0];
#pragma unroll
    for (int rb = 0; rb < RBE; ++rb) {
      const v4i lo = *(const v4i*)(ab + off_lo + rb * 2048);
      const v4i hi = *(const v4i*)(ab + off_hi + rb * 2048);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf_of(wlo[slot][cb]), bf_of(lo), acc[rb][cb], 0, 0, 0);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf_of(whi[slot][cb]), bf_of(hi), acc[rb][cb], 0, 0, 0);
    }
  };

  // One step: publish its activations, refill the ring, multiply.  LDS slot ks&1 was last read two steps ago,
  // before the previous barrier.
  auto step = [&](int ks, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    commit(ks, s_c);
    barrier_lds();
    issue(ks + S - 1, IntC<(s + S - 1) % S>{});
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this step's matrix instructions
    compute(ks, s_c);
  };

  static_for<0, S - 1>([&](auto s_c) { issue(decltype(s_c)::value, s_c); });
  const int nfull = KS / S;
  for (int g = 0; g < nfull; ++g) static_for<0, S>([&](auto s_c) { step(g * S + decltype(s_c)::value, s_c); });
  static_for<0, S>([&](auto s_c) {
    const int ks = nfull * S + decltype(s_c)::value;
    if (ks < KS) step(ks, s_c);
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
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(const GemmArgs a) {
  using C = Bf16Cfg<RB, S>;
  __shared__ __attribute__((aligned(1024))) Bf16Smem<RB, S> sm;
  __shared__ SchedSmem s_sched;
  const Sched sc{&s_sched};
  sched_build<C::BM>(a, sc);
  const Walk walk = sched_walk(s_sched.total);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  constexpr int RH = (RB + 1) / 2;  // the shorter tile height
  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const Unit u = sched_unit<C::BM>(a, sc, v);
    if (RB > 1 && u.mrows <= 16 * RH) bf16_unit<RB, S, RH>(a, u, sm, wv, lane);
    else bf16_unit<RB, S, RB>(a, u, sm, wv, lane);
  }
}

template <int RB, int S>
static hipError_t launch_bf16(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  gemm_bf16_kernel<RB, S><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs& a, int expected_m, hipStream_t s) {
  const int em = expected_m > 0 ? expected_m : (a.masked ? a.max_m : 64);
  if (em <= 16) return launch_bf16<1, 8>(a, s);
  return launch_bf16<4, 4>(a, s);
}

}  // namespace moe
