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
//    compiler's wait counts stay exact.  Each wave's weight scale of a K block
//    (one per 128 columns) is loaded into the ring with the block's weights.
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

  // weight bytes: uniform expert base + 32-bit lane offset (columns clamped for an idle wave).
  // Row-major: column n's K block at n*K + 128kb, halves 64 B apart.  Packed
  // (moe_pack_weight_fp8): the 16-column block's K block is 2 KB at
  // (kb*(N/16) + n/16)*2048, lane L's 16 bytes at 16L, halves 1 KB apart.
  const uint8_t* wbase = a.W + (int64_t)u.e * N * K;
  const uint32_t wstep = a.wpacked ? (uint32_t)N * 128u : 128u;  // bytes per K block
  const uint32_t whalf = a.wpacked ? 1024u : 64u;
  uint32_t woff[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    int n = ncol0 + 16 * cb + l16;
    if (n >= N) n = N - 1;
    woff[cb] = a.wpacked ? (uint32_t)(n / 16) * 2048u + 16u * lane : (uint32_t)n * (uint32_t)K + 16u * lg;
  }
  // this wave's 128-column block of weight scales: one per K block, loaded with the block's weights
  const float* sw_ptr = (const float*)a.SW + ((int64_t)u.e * NB + (wave_on ? ncol0 : 0) / 128) * KB;
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
  float sr[S], swr[S];
  v4f acc[RBE][CB];
#pragma unroll
  for (int rb = 0; rb < RBE; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int ks_req, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const int ks = min(ks_req, KB - 1);
    const uint32_t koff = (uint32_t)ks * 128u, wkoff = (uint32_t)ks * wstep;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const v4i* wl = (const v4i*)(wbase + (woff[cb] + wkoff));
      const v4i* wh = (const v4i*)(wbase + (woff[cb] + wkoff + whalf));
      v4i lo, hi;
      if constexpr (RB == 1) {
        // decode-sized units: an expert's rows fit one unit, so each weight byte is read once and
        // streams past the caches (5% faster on the DeepSeek-V3-shaped decode than cached loads)
        lo = __builtin_nontemporal_load(wl);
        hi = __builtin_nontemporal_load(wh);
      } else {
        lo = *wl;
        hi = *wh;
      }
      wf[slot][cb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < C::kApw; ++i) ar[slot][i] = *(const v4i*)(abase + (aoff[i] + koff));
    sr[slot] = sarow[ks];
    swr[slot] = sw_ptr[ks];
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
    const int swe = (int)(__float_as_uint(swr[slot]) >> 23);
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
  __shared__ SchedSmem s_sched;

  const Sched sc{&s_sched};
  sched_build<C::BM>(a, sc);
  const Walk walk = sched_walk(s_sched.total);
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
// Tall tiles (prefill): up to 192 or 256 rows x 256 columns per unit, 4 waves,
// each owning 64 columns and all 6 or 8 row tiles of 32 (one wave per SIMD:
// the 192 or 256 accumulators fill the AGPRs), v_mfma_scale_f32_32x32x64_f8f6f4.
//  * Weights are private to a wave and stream from HBM straight into a 4-deep
//    register ring; activations are shared and copied global->LDS
//    (global_load_lds) into a 4-deep LDS ring.  K step ks issues the loads of
//    block ks + 2; the barrier that publishes block ks + 1 sits before the
//    step's last row tile, so the next block's first fragments are read
//    behind that tile's matrix instructions.
//  * Scales ride the same pipeline, so a unit starts without any staging
//    round trip: every 4 K blocks one 16-byte global_load_lds per lane copies
//    the next 4 fp32 row scales of 256 rows into one of two LDS group buffers
//    (a 4-byte copy per block would cost as many cache-line requests as the
//    activations themselves), each wave loads its weight scale for the block
//    into a register ring, and the E8M0 exponent is the fp32 pattern shifted
//    right by 23.  This needs K/128 to be a multiple of 4 and SFA 16-byte
//    aligned; other calls take the 64-row tile.
//  * The K loop and the epilogue are written out in assembly
//    (gen_fp8_asm.py -> gemm_fp8_tall_loop.inc), once per row-tile count, so
//    no branch sits between matrix instructions: fixed registers for the
//    accumulators and the weight ring, loads spread one per matrix
//    instruction, exact vmcnt waits, a unit computes max(2, ceil(rows/32))
//    row tiles (the surplus rows repeat the last valid row and are never
//    stored), and v_cvt_pk_bf16_f32 (round to nearest even).  The epilogue
//    runs inside the last K block, which issues none of the unit's own
//    loads: while row tile j is multiplied, row tile j - 1 is converted and
//    staged through the wave's 4 KB of the idle ring slot 2 and row tile
//    j - 2 is stored as whole 128-byte rows; only the last row tile is stored
//    after the loop.  Meanwhile the next unit's first two K blocks are issued
//    (see fp8_unit_tall).
//  * The 192-row tile's weight loads are nontemporal: it serves experts of
//    about one chunk, whose weight bytes are read by one unit each (2-4%
//    faster on DeepSeek-V3-shaped prefill); the 256-row tile's are not,
//    since the many chunks of its experts re-read the weights from L2.
#include "gemm_fp8_tall_loop.inc"

template <int ROWS>
struct TallCfg;
template <>
struct TallCfg<192> {
  static constexpr int S = MOE_FP8_TALL192_S, kApw = MOE_FP8_TALL192_APW, kSlot = MOE_FP8_TALL192_SLOT,
                       kSlotA = MOE_FP8_TALL192_SLOT_A, kScOff = MOE_FP8_TALL192_SC_OFF,
                       kLds = MOE_FP8_TALL192_LDS;
};
template <>
struct TallCfg<256> {
  static constexpr int S = MOE_FP8_TALL256_S, kApw = MOE_FP8_TALL256_APW, kSlot = MOE_FP8_TALL256_SLOT,
                       kSlotA = MOE_FP8_TALL256_SLOT_A, kScOff = MOE_FP8_TALL256_SC_OFF,
                       kLds = MOE_FP8_TALL256_LDS;
};

template <int ROWS>
struct Fp8TallSmem {
  // S ring slots of activation rows (128 B each, 16-B chunks XOR-swizzled), then two row-scale group
  // buffers (row r's 4 fp32 scales at 16 r)
  uint8_t b[TallCfg<ROWS>::kLds];
};
static_assert(MOE_FP8_TALL_SCALE_ROWS == 256, "row scales: 4 waves x 64 lanes");
static_assert(MOE_FP8_TALL_SCALE_GROUP == 4, "a row-scale copy covers 4 K blocks (16 bytes)");
static_assert(TallCfg<192>::kSlotA == 192 * 128 && TallCfg<192>::kApw * 32 == 192, "192-row slots");
static_assert(TallCfg<256>::kSlotA == 256 * 128 && TallCfg<256>::kApw * 32 == 256, "256-row slots");
// the SwiGLU loops share the register and LDS layout of the plain ones
static_assert(MOE_SWIGLU_TALL192_LDS == MOE_FP8_TALL192_LDS && MOE_SWIGLU_TALL192_SLOT == MOE_FP8_TALL192_SLOT &&
                  MOE_SWIGLU_TALL192_S == MOE_FP8_TALL192_S && MOE_SWIGLU_TALL192_APW == MOE_FP8_TALL192_APW,
              "SwiGLU 192-row layout");
static_assert(MOE_SWIGLU_TALL256_LDS == MOE_FP8_TALL256_LDS && MOE_SWIGLU_TALL256_SLOT == MOE_FP8_TALL256_SLOT &&
                  MOE_SWIGLU_TALL256_S == MOE_FP8_TALL256_S && MOE_SWIGLU_TALL256_APW == MOE_FP8_TALL256_APW,
              "SwiGLU 256-row layout");
// SwiGLU staging: row m's 128 gate and 128 up bf16 values at 512 m, over the ring (which ends at the scales)
static_assert(TallCfg<192>::kScOff == 192 * 512 && TallCfg<256>::kScOff == 256 * 512, "SwiGLU staging fits");

__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

#define MOE_TALL_ASM(LOOP, AO_OUTS, CLOBBERS)                                                                     \
  asm volatile(LOOP                                                                                             \
               : [wo0] "+v"(wo[0]), [wo1] "+v"(wo[1]), AO_OUTS,                                                    \
                 [so] "+v"(so), [wso] "+v"(wso), [doff] "+v"(doff), [ks] "=&s"(ks), [q] "=&s"(q), [t] "=&s"(t),  \
                 [inc] "=&s"(inc), [inc4] "=&s"(inc4), [sv] "=&s"(sv), [m0v] "+{m0}"(m0v), [msg] "+s"(msg)                         \
               : [wb] "s"(wb), [ab] "s"(ab), [sb] "s"(sb), [swb] "s"(swb), [ma] "s"(ma),                       \
                 [a00] "v"(af[0]), [a01] "v"(af[1]), [a10] "v"(af[2]), [a11] "v"(af[3]), [sadr] "v"(sadr),        \
                 [db] "s"(db), [dstep] "s"(dstep), [kb] "s"(kb),                                                 \
                 [rbe] "s"(rbe), [mrows] "s"(mrows), [won] "s"(wons), [wm] "s"(wm), [wstep] "s"(wstep),           \
                 [l8] "v"(l8), [epb] "v"(epb), [rb] "v"(rb)                                                      \
               : "memory", "vcc", "exec", "scc", CLOBBERS)

// SwiGLU after the up-projection's loop (SWIGLU units): the unit's gate and up values, rounded to bf16, are in
// LDS (row m at 512 m: gate values 0 .. 127 of the unit's 128 outputs, then up values; 16-byte chunk c at
// position c ^ (m & 31)).  16 lanes per row, 4 rows per wave: each lane takes 8 consecutive outputs, and the
// row's 128 outputs are one 1x128 quantisation block (column tile n0 / 256).  Rows of the computed row tiles
// past the unit's end are read (they repeat its last row) but not stored.  The closing barrier keeps the next
// unit's copies into the ring behind these reads.
// The unit is passed as wave-uniform values (SGPRs), since every VGPR outside the loop's own is scarce across it.
// The plain tall loops also take the next unit's copy offsets and bases, whether this unit's first copies were
// issued by the previous unit (pfd) and whether a next unit follows (hasnext).
#define MOE_TALL_XPF_ASM(LOOP, AO_OUTS, CLOBBERS)                                                      \
  asm volatile(LOOP                                                                                             \
               : [wo0] "+v"(wo[0]), [wo1] "+v"(wo[1]), AO_OUTS,                                                    \
                 [so] "+v"(so), [wso] "+v"(wso), [doff] "+v"(doff), [ks] "=&s"(ks), [q] "=&s"(q), [t] "=&s"(t),  \
                 [inc] "=&s"(inc), [inc4] "=&s"(inc4), [sv] "=&s"(sv), [m0v] "+{m0}"(m0v), [msg] "+s"(msg),       \
                 [nso] "+v"(nso), [uo0] "+v"(uo0), [cc] "+v"(cc), [nwo0] "+v"(nwo[0]), [nwo1] "+v"(nwo[1]),      \
                 [nwso] "+v"(nwso)                                                                               \
               : [wb] "s"(wb), [ab] "s"(ab), [sb] "s"(sb), [swb] "s"(swb), [ma] "s"(ma),                       \
                 [a00] "v"(af[0]), [a01] "v"(af[1]), [a10] "v"(af[2]), [a11] "v"(af[3]), [sadr] "v"(sadr),        \
                 [db] "s"(db), [dstep] "s"(dstep), [kb] "s"(kb),                                                 \
                 [rbe] "s"(rbe), [mrows] "s"(mrows), [won] "s"(wons), [wm] "s"(wm), [wstep] "s"(wstep),           \
                 [l8] "v"(l8), [epb] "v"(epb), [rb] "v"(rb), [nab] "s"(nab), [nsb] "s"(nsb),                      \
                 [nlim] "s"(nlim), [fl] "s"(flags), [nwb] "s"(nwb), [nswb] "s"(nswb)                              \
               : "memory", "vcc", "exec", "scc", CLOBBERS)

template <int ROWS>
__device__ __forceinline__ void swiglu_unit_rows(const GemmArgs& a, const Fp8TallSmem<ROWS>& sm, int row0,
                                                 int mrows, int nt, int rbe) {
  // (the lane id through a volatile statement: nothing of this pass is hoisted out of the unit loop to stay live
  // across the loop's assembly, where the compiler has few registers)
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int I = a.N / 2, ib = I / 128, sub = lane & 15, wv = uniform(threadIdx.x >> 6);
#pragma unroll 2
  for (int m0 = 0; m0 < 32 * rbe; m0 += 16) {  // (2 rbe iterations; two rows' chains interleave: 4 was slower)
    const int m = m0 + 4 * wv + (lane >> 4), sw = m & 31;
    const v4i g = *(const v4i*)&sm.b[m * 512 + 16 * (sub ^ sw)];
    const v4i up = *(const v4i*)&sm.b[m * 512 + 16 * ((16 + sub) ^ sw)];
    uint2 o;
    const int e = swiglu_quant16(g, up, &o);
    if (m < mrows) {
      const int64_t row = (int64_t)row0 + m;
      *(uint2*)(a.Q + row * I + 128 * nt + 8 * sub) = o;
      if (sub == 0) a.SQ[row * ib + nt] = pow2f(e);
    }
  }
  __syncthreads();
}

// Plain units (not SWIGLU) pipeline across units: the last K block of unit u issues the activation copies of
// K blocks 0 and 1 of the next unit nu (and its first row-scale group) into the ring slots 0 and 1, idle by
// then, and u's loop ends by issuing nu's weights and weight scales of those blocks into the ring registers,
// so nu's loop starts with its first two K blocks in flight; msgs carries the row-scale group buffer across
// units.  pfd: u's first loads were issued that way; hasnext: nu is a real unit (else nu is u itself, its
// copies repeat u's own harmlessly and the loop waits for them instead of issuing weights).
template <int ROWS, bool PACKED, bool SWIGLU>
__device__ __forceinline__ void fp8_unit_tall(const GemmArgs& a, const Unit& u, Fp8TallSmem<ROWS>& sm, int wv,
                                              int lane, const Unit& nu, int pfd, int hasnext, uint32_t& msgs) {
  constexpr int kTApw = TallCfg<ROWS>::kApw, kScOff = TallCfg<ROWS>::kScOff, kSlot = TallCfg<ROWS>::kSlot;
  const int l32 = lane & 31, hh = lane >> 5;  // operand row and K half of this lane
  const int K = a.K, N = a.N, KB = K / 128, NB = N / 128;
  // SwiGLU: the unit's 128 outputs are gate columns n0 / 2 .. + 127 (waves 0, 1) and the up columns N / 2
  // further (waves 2, 3); every wave has columns (N / 2 is a multiple of 128)
  const int ncol0 = SWIGLU ? (wv >= 2 ? N / 2 : 0) + u.n0 / 2 + 64 * (wv & 1) : u.n0 + 64 * wv;
  const int won = ncol0 < N ? 1 : 0;
  const int ncl = won ? ncol0 : N - 64;  // an idle wave re-reads valid columns and stores nothing

  // weights: column tile c (32 columns) of this wave; see the operand notes in gen_fp8_asm.py
  const uint64_t wb = uniform_u64((uint64_t)(a.W + (int64_t)u.e * N * K));
  const int wstep = uniform(PACKED ? 128 * N : 128);  // weight bytes per K block
  const auto wcol = [&](int col, int c) {
    return PACKED ? (uint32_t)((col + 32 * c) / 16 + l32 / 16) * 2048u + (uint32_t)((l32 & 15) + 32 * hh) * 16u
                  : (uint32_t)(col + 32 * c + l32) * (uint32_t)K + 32u * hh;
  };
  uint32_t wo[2], nwo[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) wo[c] = wcol(ncl, c) + (pfd ? 2u * (uint32_t)wstep : 0u);  // (pfd: from block 2)
  // the next unit's weights, loaded at the end of this unit's loop (an idle wave's columns clamped as above)
  const int nncol0 = nu.n0 + 64 * wv, nncl = nncol0 < N ? nncol0 : N - 64;
#pragma unroll
  for (int c = 0; c < 2; ++c) nwo[c] = SWIGLU ? 0u : wcol(nncl, c);
  const uint64_t nwb = SWIGLU ? 0 : uniform_u64((uint64_t)(a.W + (int64_t)nu.e * N * K));
  const uint64_t nswb =
      SWIGLU ? 0 : uniform_u64((uint64_t)((const float*)a.SW + ((int64_t)nu.e * NB + nncl / 128) * KB));
  uint32_t nwso = 0;
  const uint64_t ab = uniform_u64((uint64_t)(a.A + (int64_t)u.row0 * K));
  uint32_t ao[kTApw];
  // (copies of K blocks 0 and 1 already issued: the offsets start at block 2)
  const uint32_t a_skip = pfd ? 256u : 0u;
#pragma unroll
  for (int i = 0; i < kTApw; ++i) {
    const int r = 8 * (4 * i + wv) + (lane >> 3);  // tile row this lane copies (copy i of the wave)
    const int c = (lane & 7) ^ ((r >> 1) & 7);     // its chunk, landing at position lane & 7 (c = cc / 16 below)
    ao[i] = (uint32_t)min(r, u.mrows - 1) * (uint32_t)K + 16u * c + a_skip;
  }
  // the next unit's copies (the loop derives their offsets): row 8 wv + lane / 8 of copy 0, unclamped
  // (cc, uo0, nso: in/out operands of the loop, so that no output can share their registers)
  uint32_t cc = SWIGLU ? 0u : 16u * (uint32_t)((lane & 7) ^ ((4 * wv + (lane >> 4)) & 7));
  uint32_t uo0 = SWIGLU ? 0u : (uint32_t)(8 * wv + (lane >> 3)) * (uint32_t)K + cc;
  const int nlim = SWIGLU ? 0 : uniform((nu.mrows - 1) * K);
  const uint64_t nab = SWIGLU ? 0 : uniform_u64((uint64_t)(a.A + (int64_t)nu.row0 * K));
  // row scales: lane copies row 64 wv + lane (the unit's last row past its end), 16 bytes per 4 K blocks
  const uint64_t sb = uniform_u64((uint64_t)(a.SFA + (int64_t)u.row0 * KB));
  uint32_t so = (uint32_t)min(64 * wv + lane, u.mrows - 1) * (uint32_t)(KB * 4) + (pfd && KB > 4 ? 16u : 0u);
  const uint64_t nsb = SWIGLU ? 0 : uniform_u64((uint64_t)(a.SFA + (int64_t)nu.row0 * KB));
  uint32_t nso = SWIGLU ? 0u : (uint32_t)min(64 * wv + lane, nu.mrows - 1) * (uint32_t)(KB * 4);
  // weight scale of this wave's 64 columns (one 128-column block), the same address in every lane
  const uint64_t swb = uniform_u64((uint64_t)((const float*)a.SW + ((int64_t)u.e * NB + ncl / 128) * KB));
  uint32_t wso = pfd ? 8u : 0u;

  // fragment reads: row m at m*128, chunk c at position c ^ ((m >> 1) & 7); lane (row l32, half hh) reads
  // chunks 4 kk + 2 hh + p for the halves kk and pieces p of the K block
  const int fsw = (l32 >> 1) & 7;
  const uint32_t abase = lds_offset(&sm.b[0]);
  uint32_t af[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) af[i] = abase + l32 * 128 + 16 * ((4 * (i >> 1) + 2 * hh + (i & 1)) ^ fsw);
  const uint32_t ma = (uint32_t)uniform((int)lds_offset(&sm.b[wv * 1024]));  // copy i at + 4096 i
  // row-scale group buffer of the next group copy (0 or 1, 4 KB apart); the unit's first group is in the one
  // msg points at, or (pfd) was copied there before the previous unit's copy toggled msg
  const uint32_t msg0 = (uint32_t)uniform((int)lds_offset(&sm.b[kScOff + wv * 1024]));
  uint32_t msg = SWIGLU ? msg0 : (uint32_t)uniform((int)msgs);
  const uint32_t sbuf = (pfd ? msg ^ 4096u : msg) - msg0;
  const uint32_t sadr = abase + kScOff + 16 * l32 + sbuf;  // row scale of row tile j, block s: +512 j + 4 s
  // epilogue: one 32-row tile of the wave's bf16 rows at a time goes through its own 4 KB of ring slot 2
  // (slots 0 and 1 receive the next unit's copies meanwhile; row m at m*128, 16-byte chunk c at position
  // c ^ (m & 7)); each lane writes 8 bytes of row l32 (epb: chunk 0's address, including the lane's half) and
  // reads back 16 bytes (chunk lane & 7) of row lane >> 3 of every 8-row group, stored as whole 128-byte rows
  // (SwiGLU: epb is this lane's 8 bytes of chunk 8 wv of row l32 of the staged bf16 rows, see swiglu_unit_rows)
  const uint32_t stg = abase + (SWIGLU ? 0u : 2u * kSlot);
  const uint32_t epb = SWIGLU ? abase + (uint32_t)(l32 * 512 + 16 * ((8 * wv) ^ l32) + 8 * hh)
                              : stg + (uint32_t)(wv * 4096 + l32 * 128 + 16 * (l32 & 7) + 8 * hh);
  const int l8 = lane >> 3;
  const uint32_t rb = stg + (uint32_t)(wv * 4096 + l8 * 128 + 16 * ((lane & 7) ^ (l8 & 7)));
  const uint64_t wm = uniform_u64(won ? ~0ull : 0ull);  // exec mask of the stores: none for an idle wave
  const uint64_t db = SWIGLU ? 0 : uniform_u64((uint64_t)(a.D + (int64_t)u.row0 * N));  // (SwiGLU: no D)
  uint32_t doff = (uint32_t)(l8 * N + ncol0 + 8 * (lane & 7)) * 2u;
  const int dstep = uniform(16 * N);  // output bytes between 8-row groups
  // row tiles computed: at least 2, so the barrier that publishes the next K block (after the fragments of
  // the second-to-last row tile's successor are read) has a place in every step
  const int rbe = uniform(max(2, (u.mrows + 31) / 32));
  const int kb = uniform(KB), mrows = uniform(u.mrows), wons = uniform(won);
  const int flags = uniform(pfd | (hasnext << 1));  // bit 0: pfd, bit 1: hasnext
  const int row0 = uniform(u.row0), nt = uniform(u.n0 / 256);  // (SwiGLU, after the loop)
  int ks, q, t, inc, inc4, m0v = 0;
  uint64_t sv;
  if constexpr (SWIGLU) {
    if constexpr (ROWS == 192) {
      if constexpr (PACKED)
        MOE_TALL_ASM(MOE_SWIGLU_TALL192_LOOP_PACKED, MOE_SWIGLU_TALL192_AO_OUTS, MOE_SWIGLU_TALL192_CLOBBERS);
      else
        MOE_TALL_ASM(MOE_SWIGLU_TALL192_LOOP, MOE_SWIGLU_TALL192_AO_OUTS, MOE_SWIGLU_TALL192_CLOBBERS);
    } else {
      if constexpr (PACKED)
        MOE_TALL_ASM(MOE_SWIGLU_TALL256_LOOP_PACKED, MOE_SWIGLU_TALL256_AO_OUTS, MOE_SWIGLU_TALL256_CLOBBERS);
      else
        MOE_TALL_ASM(MOE_SWIGLU_TALL256_LOOP, MOE_SWIGLU_TALL256_AO_OUTS, MOE_SWIGLU_TALL256_CLOBBERS);
    }
    swiglu_unit_rows<ROWS>(a, sm, row0, mrows, nt, rbe);
  } else if constexpr (ROWS == 192) {
    if constexpr (PACKED)
      MOE_TALL_XPF_ASM(MOE_FP8_TALL192_LOOP_PACKED, MOE_FP8_TALL192_AO_OUTS, MOE_FP8_TALL192_CLOBBERS);
    else
      MOE_TALL_XPF_ASM(MOE_FP8_TALL192_LOOP, MOE_FP8_TALL192_AO_OUTS, MOE_FP8_TALL192_CLOBBERS);
  } else {
    if constexpr (PACKED)
      MOE_TALL_XPF_ASM(MOE_FP8_TALL256_LOOP_PACKED, MOE_FP8_TALL256_AO_OUTS, MOE_FP8_TALL256_CLOBBERS);
    else
      MOE_TALL_XPF_ASM(MOE_FP8_TALL256_LOOP, MOE_FP8_TALL256_AO_OUTS, MOE_FP8_TALL256_CLOBBERS);
  }
  if constexpr (!SWIGLU) msgs = msg;
}

template <int ROWS>
__global__ __launch_bounds__(256, 1) void gemm_fp8_tall_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) Fp8TallSmem<ROWS> sm;
  __shared__ SchedSmem s_sched;
  const Sched sc{&s_sched};
  sched_build<ROWS>(a, sc);
  const Walk walk = sched_walk(s_sched.total);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  // each unit's last K block issues the next unit's first activation copies (see fp8_unit_tall)
  uint32_t msgs = (uint32_t)uniform((int)lds_offset(&sm.b[TallCfg<ROWS>::kScOff + wv * 1024]));
  int pfd = 0;
  Unit u;
  if (walk.first < walk.end) u = sched_unit<ROWS>(a, sc, walk.first);
  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const int hasnext = v + walk.stride < walk.end;
    const Unit nu = hasnext ? sched_unit<ROWS>(a, sc, v + walk.stride) : u;
    if (a.wpacked) fp8_unit_tall<ROWS, true, false>(a, u, sm, wv, lane, nu, pfd, hasnext, msgs);
    else fp8_unit_tall<ROWS, false, false>(a, u, sm, wv, lane, nu, pfd, hasnext, msgs);
    u = nu;
    pfd = hasnext;
  }
}

// The up-projection with SwiGLU and its 1x128 requantisation in the epilogue (a separate kernel, so the plain
// GEMM's code is untouched): the same tall units over N = 2I columns, with Q / SQ written instead of D.
template <int ROWS>
__global__ __launch_bounds__(256, 1) void gemm_fp8_swiglu_tall_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) Fp8TallSmem<ROWS> sm;
  __shared__ SchedSmem s_sched;
  const Sched sc{&s_sched};
  sched_build<ROWS>(a, sc);
  const Walk walk = sched_walk(s_sched.total);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const Unit u = sched_unit<ROWS>(a, sc, v);
    uint32_t msgs = 0;  // (SwiGLU units start at group buffer 0)
    if (a.wpacked) fp8_unit_tall<ROWS, true, true>(a, u, sm, wv, lane, u, 0, 0, msgs);
    else fp8_unit_tall<ROWS, false, true>(a, u, sm, wv, lane, u, 0, 0, msgs);
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

template <int ROWS, bool SWIGLU = false>
static hipError_t launch_fp8_tall(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  if (SWIGLU) gemm_fp8_swiglu_tall_kernel<ROWS><<<grid, 256, 0, s>>>(a);
  else gemm_fp8_tall_kernel<ROWS><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const GemmArgs& a, int expected_m, hipStream_t s) {
  // Tile height from the expected rows per active expert: decode-sized
  // segments stream the weights through a register ring (short tiles),
  // prefill segments use the tall tiles (192 or 256 rows).  The decode ring
  // keeps two K blocks in flight per wave (32 KB per CU per block): deeper
  // rings (3 to 7 blocks) were 1-3% slower on the DeepSeek-V3-shaped decode,
  // one block 7% slower -- a plain streaming read is also fastest with about
  // 32 KB in flight per CU.
  const int em = expected_m > 0 ? expected_m : (a.masked ? a.max_m : 256);
  if (em <= 16) return launch_fp8<1, 3, 4>(a, s);
  // the tall tile copies 4 K blocks of row scales per 16-byte load
  const bool tall_ok = (a.K / 128) % MOE_FP8_TALL_SCALE_GROUP == 0 && (((uintptr_t)a.SFA) & 15) == 0;
  if (em <= 64 || !tall_ok) return launch_fp8<4, 6, 4>(a, s);
  // 256-row tiles read each weight tile once per 256 rows instead of 192 but
  // copy 256 activation rows per K block whatever the unit holds: worth it
  // once a typical expert fills them
  if (em >= 256) return launch_fp8_tall<256>(a, s);
  return launch_fp8_tall<192>(a, s);
}

hipError_t launch_gemm_fp8_swiglu(const GemmArgs& a, int expected_m, hipStream_t s) {
  // tall tiles only (the caller checked K / 128 % 4 == 0 and the 16-byte row-scale alignment they need); the
  // tile height as for the plain GEMM
  const int em = expected_m > 0 ? expected_m : (a.masked ? a.max_m : 256);
  if (em >= 256) return launch_fp8_tall<256, true>(a, s);
  return launch_fp8_tall<192, true>(a, s);
}

}  // namespace moe
