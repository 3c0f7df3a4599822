// gemm_bf16.hip -- BF16 grouped GEMM for gfx950 (contiguous and masked layouts).
//
// D[p, n] = bf16( sum_k a[p,k] * w[e,n,k] ), fp32 accumulation
// (AsymGEMM README, "API Reference": BF16 m_grouped contiguous and masked
// grouped GEMMs, NT operands, bf16 output; rainlin, "GEMM 执行方式", sec. 4.6:
// the BF16 contiguous grouped GEMM called on the packed segments.)
//
// Short tiles (decode, and rows that fill no tall tile): the same design as the
// FP8 short tiles (gemm_fp8.hip), on the bf16 matrix instruction and without
// scales:
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
  // Packed (moe_pack_weight_bf16): the weight bytes in moe_pack_weight_fp8's order with 2K bytes per row, i.e.
  // step ks of the 16-column block of column n is 2 KB at (ks*(N/16) + n/16)*2048, the lane's 16 bytes at
  // 16 lane and its second piece 1 KB further.
  using C = Bf16Cfg<RB, S>;
  const int l16 = lane & 15, lg = lane >> 4;
  const int K = a.K, N = a.N, KS = K / 64;
  const uint32_t rowb = (uint32_t)K * 2u;  // bytes per row of A and of W
  const int ncol0 = u.n0 + 64 * wv;        // this wave's first column
  const bool wave_on = ncol0 < N;

  // weights: column n's step ks is 128 bytes at n*2K + 128 ks; the lane's halves at +16 lg and +64 + 16 lg
  const uint8_t* wbase = a.W + (int64_t)u.e * N * rowb;
  const uint32_t wstep = a.wpacked ? (uint32_t)N * 128u : 128u;  // bytes per step
  const uint32_t whalf = a.wpacked ? 1024u : 64u;
  uint32_t woff[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    int n = ncol0 + 16 * cb + l16;
    if (n >= N) n = N - 1;  // an idle wave re-reads valid columns and stores nothing
    woff[cb] = a.wpacked ? (uint32_t)(n / 16) * 2048u + 16u * lane : (uint32_t)n * rowb + 16u * lg;
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
    const uint32_t ks = (uint32_t)min(ks_req, KS - 1), koff = ks * 128u;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const uint8_t* wp = wbase + (woff[cb] + ks * wstep);
      if constexpr (RB == 1) {
        // decode-sized units: an expert's rows fit one unit, so each weight byte is read once
        wlo[slot][cb] = __builtin_nontemporal_load((const v4i*)wp);
        whi[slot][cb] = __builtin_nontemporal_load((const v4i*)(wp + whalf));
      } else {
        wlo[slot][cb] = *(const v4i*)wp;
        whi[slot][cb] = *(const v4i*)(wp + whalf);
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

// ----------------------------------------------------------------------------
// Tall tiles (prefill): 192 or 256 rows x 256 columns per unit, the FP8 tall
// tiles' generated loop (gen_fp8_asm.py, the bf16 configurations) with each
// scaled 32x32x64 FP8 instruction replaced by two v_mfma_f32_32x32x16_bf16 on
// the two 16-byte pieces of each operand -- a 128-byte step of every row is
// the same bytes and the same matrix-core cycles as an FP8 K block -- and no
// scales.  Weights stream into the 4-deep register ring, activations into the
// 4-deep LDS ring (global_load_lds), the epilogue runs inside the last step.
// Needs K/64 to be a multiple of 4 (the loop body is 4 steps).
#include "gemm_fp8_tall_loop.inc"

template <int ROWS>
struct Bf16TallCfg;
template <>
struct Bf16TallCfg<192> {
  static constexpr int kApw = MOE_BF16_TALL192_APW, kLds = MOE_BF16_TALL192_LDS;
};
template <>
struct Bf16TallCfg<256> {
  static constexpr int kApw = MOE_BF16_TALL256_APW, kLds = MOE_BF16_TALL256_LDS;
};
static_assert(MOE_BF16_TALL192_S == 4 && MOE_BF16_TALL256_S == 4, "4-step loop body");
static_assert(MOE_BF16_TALL192_SLOT_A == 192 * 128 && MOE_BF16_TALL256_SLOT_A == 256 * 128, "128-byte rows per slot");

__device__ __forceinline__ uint64_t uniform_u64_bf(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// The generated loop names the FP8 tile's scale operands too; the bf16 loop never uses them (dummies).
#define MOE_BF16_TALL_ASM(LOOP, AO_OUTS, CLOBBERS)                                                                \
  asm volatile(LOOP                                                                                             \
               : [wo0] "+v"(wo[0]), [wo1] "+v"(wo[1]), AO_OUTS,                                                    \
                 [so] "+v"(so), [wso] "+v"(wso), [doff] "+v"(doff), [ks] "=&s"(ks), [q] "=&s"(q), [t] "=&s"(t),  \
                 [inc] "=&s"(inc), [inc4] "=&s"(inc4), [sv] "=&s"(sv), [m0v] "+{m0}"(m0v), [msg] "+s"(msg)         \
               : [wb] "s"(wb), [ab] "s"(ab), [sb] "s"(sb), [swb] "s"(swb), [ma] "s"(ma),                       \
                 [a00] "v"(af[0]), [a01] "v"(af[1]), [a10] "v"(af[2]), [a11] "v"(af[3]), [sadr] "v"(sadr),        \
                 [db] "s"(db), [dstep] "s"(dstep), [kb] "s"(kb),                                                 \
                 [rbe] "s"(rbe), [mrows] "s"(mrows), [won] "s"(wons), [wm] "s"(wm), [wstep] "s"(wstep),           \
                 [l8] "v"(l8), [epb] "v"(epb), [rb] "v"(rb)                                                      \
               : "memory", "vcc", "exec", "scc", CLOBBERS)

template <int ROWS, bool PACKED>
__device__ __forceinline__ void bf16_unit_tall(const GemmArgs& a, const Unit& u, uint8_t* smem, int wv, int lane) {
  constexpr int kTApw = Bf16TallCfg<ROWS>::kApw;
  const int l32 = lane & 31, hh = lane >> 5;  // operand row and K half of this lane
  const int K = a.K, N = a.N, KS = K / 64;
  const uint32_t rowb = (uint32_t)K * 2u;
  const int ncol0 = u.n0 + 64 * wv;
  const int won = ncol0 < N ? 1 : 0;
  const int ncl = won ? ncol0 : N - 64;  // an idle wave re-reads valid columns and stores nothing

  // weights: column tile c (32 columns) of this wave; lane (l32, hh) reads the 32 bytes 32 hh .. 32 hh + 31 of
  // each 64-byte half kk of the step, as two 16-byte pieces (in the packed order, chunks of the 2 KB fragment)
  const uint64_t wb = uniform_u64_bf((uint64_t)(a.W + (int64_t)u.e * N * rowb));
  uint32_t wo[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    wo[c] = PACKED ? (uint32_t)((ncl + 32 * c) / 16 + l32 / 16) * 2048u + (uint32_t)((l32 & 15) + 32 * hh) * 16u
                   : (uint32_t)(ncl + 32 * c + l32) * rowb + 32u * hh;
  const int wstep = uniform(PACKED ? 128 * N : 128);  // weight bytes per step
  const uint64_t ab = uniform_u64_bf((uint64_t)(a.A + (int64_t)u.row0 * rowb));
  uint32_t ao[kTApw];
#pragma unroll
  for (int i = 0; i < kTApw; ++i) {
    const int r = 8 * (4 * i + wv) + (lane >> 3);  // tile row this lane copies (copy i of the wave)
    const int c = (lane & 7) ^ ((r >> 1) & 7);     // its chunk, landing at position lane & 7
    ao[i] = (uint32_t)min(r, u.mrows - 1) * rowb + 16u * c;
  }
  const uint64_t sb = 0, swb = 0;
  uint32_t so = 0, wso = 0;
  // fragment reads: row m at m*128, chunk c at position c ^ ((m >> 1) & 7); lane (row l32, half hh) reads chunks
  // 4 kk + 2 hh + p for the halves kk and pieces p of the step
  const int fsw = (l32 >> 1) & 7;
  const uint32_t abase = lds_offset(smem);
  uint32_t af[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) af[i] = abase + l32 * 128 + 16 * ((4 * (i >> 1) + 2 * hh + (i & 1)) ^ fsw);
  const uint32_t sadr = 0;
  const uint32_t ma = (uint32_t)uniform((int)lds_offset(smem + wv * 1024));  // copy i at + 4096 i
  uint32_t msg = 0;
  // epilogue staging, as in the FP8 tall tile (each wave's 4 KB of ring slot 0)
  const uint32_t epb = abase + (uint32_t)(wv * 4096 + l32 * 128 + 16 * (l32 & 7) + 8 * hh);
  const int l8 = lane >> 3;
  const uint32_t rb = abase + (uint32_t)(wv * 4096 + l8 * 128 + 16 * ((lane & 7) ^ (l8 & 7)));
  const uint64_t wm = uniform_u64_bf(won ? ~0ull : 0ull);
  const uint64_t db = uniform_u64_bf((uint64_t)(a.D + (int64_t)u.row0 * N));
  uint32_t doff = (uint32_t)(l8 * N + ncol0 + 8 * (lane & 7)) * 2u;
  const int dstep = uniform(16 * N);
  const int rbe = uniform(max(2, (u.mrows + 31) / 32));
  const int kb = uniform(KS), mrows = uniform(u.mrows), wons = uniform(won);
  int ks, q, t, inc, inc4, m0v = 0;
  uint64_t sv;
  if constexpr (ROWS == 192) {
    if constexpr (PACKED)
      MOE_BF16_TALL_ASM(MOE_BF16_TALL192_LOOP_PACKED, MOE_BF16_TALL192_AO_OUTS, MOE_BF16_TALL192_CLOBBERS);
    else
      MOE_BF16_TALL_ASM(MOE_BF16_TALL192_LOOP, MOE_BF16_TALL192_AO_OUTS, MOE_BF16_TALL192_CLOBBERS);
  } else {
    if constexpr (PACKED)
      MOE_BF16_TALL_ASM(MOE_BF16_TALL256_LOOP_PACKED, MOE_BF16_TALL256_AO_OUTS, MOE_BF16_TALL256_CLOBBERS);
    else
      MOE_BF16_TALL_ASM(MOE_BF16_TALL256_LOOP, MOE_BF16_TALL256_AO_OUTS, MOE_BF16_TALL256_CLOBBERS);
  }
}

template <int ROWS>
__global__ __launch_bounds__(256, 1) void gemm_bf16_tall_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sm[Bf16TallCfg<ROWS>::kLds];
  __shared__ SchedSmem s_sched;
  const Sched sc{&s_sched};
  sched_build<ROWS>(a, sc);
  const Walk walk = sched_walk(s_sched.total);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const Unit u = sched_unit<ROWS>(a, sc, v);
    if (a.wpacked) bf16_unit_tall<ROWS, true>(a, u, sm, wv, lane);
    else bf16_unit_tall<ROWS, false>(a, u, sm, wv, lane);
  }
}

template <int ROWS>
static hipError_t launch_bf16_tall(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  gemm_bf16_tall_kernel<ROWS><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
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
  const int em = expected_m > 0 ? expected_m : (a.masked ? a.max_m : 256);
  if (em <= 16) return launch_bf16<1, 3>(a, s);  // two K steps in flight per wave (as the FP8 decode tile)
  const bool tall_ok = (a.K / 64) % 4 == 0;  // the tall loop body is 4 steps
  if (em <= 64 || !tall_ok) return launch_bf16<4, 4>(a, s);
  if (em >= 256) return launch_bf16_tall<256>(a, s);
  return launch_bf16_tall<192>(a, s);
}

}  // namespace moe
