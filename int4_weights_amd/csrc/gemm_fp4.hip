// gemm_fp4.hip -- FP8 activations x MXFP4 weights grouped GEMM for gfx950, and
// the MXFP4 weight quantiser.
//
// D[p, n] = bf16( sum_k (a[p,k] * sa[p, k/128]) * (w[e,n,k] * 2^(sw[e,n,k/32] - 127)) )
// with a E4M3 (1x128 power-of-two scales, as the FP8 path) and w E2M1
// (AsymGEMM README, "API Reference": FP4 grouped GEMMs with the weights as
// (packed 4-bit data, scales); CuTeDSL bei Perplexity: MXFP4 block scaling;
// nxmr.cn DeepGEMM article, "精度与吞吐的平衡点": one FP4 operand is held to
// calc_diff < 0.01).  The weights are OCP MXFP4: E2M1 codes two per byte (the
// even k in the low nibble), one E8M0 scale byte per 32 consecutive K values of
// an output column -- the block size and scale format gfx950's scaled matrix
// instruction applies per lane, so the promotion is exact and free.
//
// Design (the FP8 short tiles of gemm_fp8.hip with the weight operand in E2M1):
//  * v_mfma_scale_f32_16x16x128_f8f6f4 with the A operand (16 weight columns)
//    in E2M1 (cbsz = 4) and the B operand (16 activation rows) in E4M3.  The
//    two formats place K differently in a lane (group lg): the E2M1 operand's
//    32 values are K = 32 lg .. 32 lg + 31 of the 128-value step, contiguous,
//    while the E4M3 operand's 32 bytes are K = 16 lg .. 16 lg + 15 and then
//    64 + 16 lg .. 64 + 16 lg + 15 (measured with one-hot activation rows, a
//    GPU test).  So a weight lane loads its 32 contiguous values -- exactly one
//    MXFP4 block, whose E8M0 byte is the lane's scale -- and the activation
//    fragment is read as those two 16-byte halves, which puts every K value at
//    the same position in both operands;
//  * weights stream from HBM into an S-deep register ring (16 bytes of codes
//    and one scale dword per lane and 16-column block), activations and their
//    row scales through two XOR-swizzled LDS slots as in the FP8 kernel;
//  * packed weights (moe_pack_weight_fp4, the form the benchmark uses): each
//    load instruction reads one contiguous 1 KB fragment of codes, and one
//    256-byte load per step gives every lane a dword with its scales for the
//    wave's four 16-column blocks, the matrix instruction's op_sel picking the
//    block's byte; row-major weights read 64 bytes of each of 16 columns per
//    instruction and a lane shifts its byte out of the block's scale dword.
#include "gemm_common.h"

namespace moe {

template <int RB, int S>
struct Fp4Cfg {
  static constexpr int BM = 16 * RB;
  static constexpr int kApw = (2 * RB + 3) / 4;  // 16-byte A loads per lane per stage (1 KB = 8 rows)
  static constexpr int kArows = 4 * 8 * kApw;
  static constexpr int kAStage = kArows * 128;
  static_assert(kArows >= BM, "A stage too small");
  static_assert(S >= 2, "ring depth");
};

template <int RB, int S>
struct Fp4Smem {
  uint8_t a[2][Fp4Cfg<RB, S>::kAStage];
  float sa[2][256];  // row scales of the stage (one per lane of the 4 waves)
};

template <int RB, int S, int RBE, bool PACKED>
__device__ __forceinline__ void fp4_unit(const GemmArgs& a, const Unit& u, Fp4Smem<RB, S>& sm, int wv, int lane) {
  using C = Fp4Cfg<RB, S>;
  const int l16 = lane & 15, lg = lane >> 4;
  const int K = a.K, N = a.N, KB = K / 128;
  const int ncol0 = u.n0 + 64 * wv;
  const bool wave_on = ncol0 < N;

  // weights: column n's step ks is 64 bytes at n*K/2 + 64 ks, the lane's 16 at + 16 lg; its scale dword (the
  // step's 4 blocks) at n*K/32 + 4 ks of the scale bytes
  // Packed (moe_pack_weight_fp4): the step's 16-column block cb is 1 KB at ((ks*(N/16) + cb)*64 + lane)*16, and
  // the step's scales of the wave's 64 columns are one dword per lane at ((ks*(N/64) + n/64)*64 + lane)*4, the
  // block of column block cb in byte cb.
  const uint8_t* wbase = a.W + (int64_t)u.e * N * (K / 2);
  const uint8_t* sbase = (const uint8_t*)a.SW + (int64_t)u.e * N * (K / 32);
  uint32_t woff[4], soff[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    int n = ncol0 + 16 * cb + l16;
    if (n >= N) n = N - 1;  // an idle wave re-reads valid columns and stores nothing
    if constexpr (PACKED) {
      woff[cb] = ((uint32_t)(n / 16) * 64u + (uint32_t)lane) * 16u;
      soff[cb] = ((uint32_t)(n / 64) * 64u + (uint32_t)lane) * 4u;  // the same for the 4 blocks
    } else {
      woff[cb] = (uint32_t)n * (uint32_t)(K / 2) + 16u * lg;
      soff[cb] = (uint32_t)n * (uint32_t)(K / 32);
    }
  }
  const uint32_t wstep = PACKED ? (uint32_t)N * 64u : 64u;     // code bytes between steps
  const uint32_t sstep = (uint32_t)N * 4u;                     // packed scale bytes between steps
  const int sshift = 8 * lg;
  const uint8_t* abase = a.A + (int64_t)u.row0 * K;
  uint32_t aoff[C::kApw];
#pragma unroll
  for (int i = 0; i < C::kApw; ++i) {
    const int q = wv * C::kApw + i;
    const int r = 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    aoff[i] = (uint32_t)min(r, u.mrows - 1) * (uint32_t)K + 16u * c;
  }
  const float* sarow = a.SFA + (int64_t)(u.row0 + min(64 * wv + lane, u.mrows - 1)) * KB;
  // fragment reads: the E4M3 operand of lane group lg is K 16 lg .. +15 (chunk lg of row m = 16 rb + l16)
  // then 64 + 16 lg .. +15 (chunk 4 + lg); chunk c sits at position c ^ ((m >> 1) & 7)
  const int fsw = (l16 >> 1) & 7;
  const int off0 = l16 * 128 + 16 * (lg ^ fsw);
  const int off1 = l16 * 128 + 16 * ((4 + lg) ^ fsw);

  v4i wq[S][4];
  uint32_t sq[S][4];
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
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const v4i* wp = (const v4i*)(wbase + (woff[cb] + (uint32_t)ks * wstep));
      if constexpr (RB == 1 && PACKED)
        wq[slot][cb] = __builtin_nontemporal_load(wp);  // decode, whole lines: each weight byte is read once
      else
        wq[slot][cb] = *wp;
      if constexpr (PACKED) {
        if (cb == 0) sq[slot][0] = *(const uint32_t*)(sbase + (soff[0] + (uint32_t)ks * sstep));
      } else {
        sq[slot][cb] = *(const uint32_t*)(sbase + (soff[cb] + 4u * (uint32_t)ks));
      }
    }
#pragma unroll
    for (int i = 0; i < C::kApw; ++i) ar[slot][i] = *(const v4i*)(abase + (aoff[i] + (uint32_t)ks * 128u));
    sr[slot] = sarow[ks];
  };

  auto commit = [&](int ks, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    uint8_t* dst = &sm.a[ks & 1][0];
#pragma unroll
    for (int i = 0; i < C::kApw; ++i) *(v4i*)(dst + (wv * C::kApw + i) * 1024 + 16 * lane) = ar[slot][i];
    sm.sa[ks & 1][64 * wv + lane] = sr[slot];
  };

  auto compute = [&](int ks, auto slot_c) {
    constexpr int slot = decltype(slot_c)::value;
    const uint8_t* ab = &sm.a[ks & 1][0];
    const float* sab = &sm.sa[ks & 1][l16];
    // scale of the lane's block: packed, byte cb of the step's dword (op_sel); otherwise the lane's byte of
    // the block's dword, shifted down
    int swe[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) swe[cb] = PACKED ? (int)sq[slot][0] : (int)((sq[slot][cb] >> sshift) & 0xffu);
#pragma unroll
    for (int rb = 0; rb < RBE; ++rb) {
      const v4i x0 = *(const v4i*)(ab + off0 + rb * 2048);
      const v4i x1 = *(const v4i*)(ab + off1 + rb * 2048);
      const v8i af = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      const int sae = (int)(__float_as_uint(sab[16 * rb]) >> 23);
      static_for<0, 4>([&](auto cb_c) {
        constexpr int cb = decltype(cb_c)::value;
        const v4i w = wq[slot][cb];
        const v8i wf = v8i{w[0], w[1], w[2], w[3], 0, 0, 0, 0};  // E2M1: the instruction reads 4 registers
        acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, af, acc[rb][cb], 4, 0, PACKED ? cb : 0,
                                                                       swe[cb], 0, sae);
      });
    }
  };

  auto step = [&](int ks, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    commit(ks, s_c);
    barrier_lds();
    issue(ks + S - 1, IntC<(s + S - 1) % S>{});
    __builtin_amdgcn_sched_barrier(0);
    compute(ks, s_c);
  };

  static_for<0, S - 1>([&](auto s_c) { issue(decltype(s_c)::value, s_c); });
  const int nfull = KB / S;
  for (int g = 0; g < nfull; ++g) static_for<0, S>([&](auto s_c) { step(g * S + decltype(s_c)::value, s_c); });
  static_for<0, S>([&](auto s_c) {
    const int ks = nfull * S + decltype(s_c)::value;
    if (ks < KB) step(ks, s_c);
  });
  barrier_lds();

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

template <int RB, int S, bool PACKED>
__global__ __launch_bounds__(256, 1) void gemm_fp4_kernel(const GemmArgs a) {
  using C = Fp4Cfg<RB, S>;
  __shared__ __attribute__((aligned(1024))) Fp4Smem<RB, S> sm;
  __shared__ SchedSmem s_sched;
  const Sched sc{&s_sched};
  sched_build<C::BM>(a, sc);
  const Walk walk = sched_walk(s_sched.total);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  constexpr int RH = (RB + 1) / 2;
  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const Unit u = sched_unit<C::BM>(a, sc, v);
    if (RB > 1 && u.mrows <= 16 * RH) fp4_unit<RB, S, RH, PACKED>(a, u, sm, wv, lane);
    else fp4_unit<RB, S, RB, PACKED>(a, u, sm, wv, lane);
  }
}

template <int RB, int S, bool PACKED>
static hipError_t launch_fp4(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  gemm_fp4_kernel<RB, S, PACKED><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Tall tiles (prefill, packed weights): 192 or 256 rows x 256 columns per
// unit, the FP8 tall tiles' generated loop (gen_fp8_asm.py, the fp4
// configurations) on v_mfma_scale_f32_32x32x64_f8f6f4 with the weights as an
// E2M1 A operand (cbsz = 4).  In that instruction a weight lane (column l32,
// half h) holds the 32 contiguous values K = 64 kk + 32 h .. +31 -- one MXFP4
// block, chunk 2 kk + h of the column's 1 KB fragment in the packed order --
// and takes its own E8M0 scale, while an E4M3 activation lane holds
// K = 64 kk + 16 h .. +15 and 64 kk + 32 + 16 h .. +15 (measured with random
// small-integer operands against an exact product), so the activation
// fragment is read as chunks 4 kk + h and 4 kk + 2 + h of the row.  Each lane
// loads the packed scale dword of its 16-column group and block 2 kk + h and
// shifts it right by 8 (l32 / 16) bits x 8, so that byte 2 ct holds the scale
// of its column in column tile ct, which op_sel picks.  Activations and their
// row scales go through the LDS ring exactly as in the FP8 tall tile.
#include "gemm_fp8_tall_loop.inc"

template <int ROWS>
struct Fp4TallCfg;
template <>
struct Fp4TallCfg<192> {
  static constexpr int kApw = MOE_FP4_TALL192_APW, kScOff = MOE_FP4_TALL192_SC_OFF, kLds = MOE_FP4_TALL192_LDS;
};
template <>
struct Fp4TallCfg<256> {
  static constexpr int kApw = MOE_FP4_TALL256_APW, kScOff = MOE_FP4_TALL256_SC_OFF, kLds = MOE_FP4_TALL256_LDS;
};
static_assert(MOE_FP4_TALL192_S == 4 && MOE_FP4_TALL256_S == 4, "4-step loop body");
static_assert(MOE_FP4_TALL192_SLOT_A == 192 * 128 && MOE_FP4_TALL256_SLOT_A == 256 * 128, "128-byte rows per slot");
static_assert(MOE_FP8_TALL_SCALE_ROWS == 256 && MOE_FP8_TALL_SCALE_GROUP == 4, "row-scale groups");

__device__ __forceinline__ uint64_t uniform_u64_f4(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

#define MOE_FP4_TALL_ASM(LOOP, AO_OUTS, CLOBBERS)                                                                 \
  asm volatile(LOOP                                                                                             \
               : [wo0] "+v"(wo[0]), [wo1] "+v"(wo[1]), AO_OUTS,                                                    \
                 [so] "+v"(so), [wso] "+v"(wso), [doff] "+v"(doff), [ks] "=&s"(ks), [q] "=&s"(q), [t] "=&s"(t),  \
                 [inc] "=&s"(inc), [inc4] "=&s"(inc4), [sv] "=&s"(sv), [m0v] "+{m0}"(m0v), [msg] "+s"(msg)         \
               : [wb] "s"(wb), [ab] "s"(ab), [sb] "s"(sb), [swb] "s"(swb), [ma] "s"(ma),                       \
                 [a00] "v"(af[0]), [a01] "v"(af[1]), [a10] "v"(af[2]), [a11] "v"(af[3]), [sadr] "v"(sadr),        \
                 [db] "s"(db), [dstep] "s"(dstep), [kb] "s"(kb), [sstep] "s"(sstep), [fsh] "v"(fsh),             \
                 [rbe] "s"(rbe), [mrows] "s"(mrows), [won] "s"(wons), [wm] "s"(wm), [wstep] "s"(wstep),           \
                 [l8] "v"(l8), [epb] "v"(epb), [rb] "v"(rb)                                                      \
               : "memory", "vcc", "exec", "scc", CLOBBERS)

template <int ROWS>
__device__ __forceinline__ void fp4_unit_tall(const GemmArgs& a, const Unit& u, uint8_t* smem, int wv, int lane) {
  constexpr int kTApw = Fp4TallCfg<ROWS>::kApw, kScOff = Fp4TallCfg<ROWS>::kScOff;
  const int l32 = lane & 31, hh = lane >> 5;  // operand row and K half of this lane
  const int K = a.K, N = a.N, KB = K / 128;
  const int ncol0 = u.n0 + 64 * wv;
  const int won = ncol0 < N ? 1 : 0;
  const int ncl = won ? ncol0 : N - 64;  // an idle wave re-reads valid columns and stores nothing

  // codes: column tile c's 16-column group (ncl + 32 c) / 16 + l32 / 16, chunk (l32 % 16) + 16 (2 kk + hh)
  const uint64_t wb = uniform_u64_f4((uint64_t)(a.W + (int64_t)u.e * N * (K / 2)));
  uint32_t wo[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    wo[c] = (uint32_t)((ncl + 32 * c) / 16 + l32 / 16) * 1024u + (uint32_t)(l32 & 15) * 16u + 256u * hh;
  const int wstep = uniform(64 * N);  // code bytes per K block
  // scales: the dword of entry (l32 % 16) + 16 (2 kk + hh) of the wave's 64-column group, bytes = the group's
  // four 16-column blocks
  const uint64_t swb = uniform_u64_f4((uint64_t)((const uint8_t*)a.SW + (int64_t)u.e * N * (K / 32)));
  uint32_t wso = (uint32_t)((ncl / 64) * 64 + (l32 & 15) + 16 * hh) * 4u;
  const int sstep = uniform(4 * N);   // scale bytes per K block
  const uint32_t fsh = 8u * (uint32_t)(l32 >> 4);
  // activations and row scales as in the FP8 tall tile
  const uint64_t ab = uniform_u64_f4((uint64_t)(a.A + (int64_t)u.row0 * K));
  uint32_t ao[kTApw];
#pragma unroll
  for (int i = 0; i < kTApw; ++i) {
    const int r = 8 * (4 * i + wv) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    ao[i] = (uint32_t)min(r, u.mrows - 1) * (uint32_t)K + 16u * c;
  }
  const uint64_t sb = uniform_u64_f4((uint64_t)(a.SFA + (int64_t)u.row0 * KB));
  uint32_t so = (uint32_t)min(64 * wv + lane, u.mrows - 1) * (uint32_t)(KB * 4);
  // fragment reads: row m at m*128, chunk c at position c ^ ((m >> 1) & 7); the E4M3 lane (row l32, half hh)
  // reads chunks 4 kk + hh + 2 p for the halves kk and pieces p of the K block
  const int fsw = (l32 >> 1) & 7;
  const uint32_t abase = lds_offset(smem);
  uint32_t af[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) af[i] = abase + l32 * 128 + 16 * ((4 * (i >> 1) + hh + 2 * (i & 1)) ^ fsw);
  const uint32_t sadr = abase + kScOff + 16 * l32;
  const uint32_t ma = (uint32_t)uniform((int)lds_offset(smem + wv * 1024));  // copy i at + 4096 i
  uint32_t msg = (uint32_t)uniform((int)lds_offset(smem + kScOff + wv * 1024));
  const uint32_t epb = abase + (uint32_t)(wv * 4096 + l32 * 128 + 16 * (l32 & 7) + 8 * hh);
  const int l8 = lane >> 3;
  const uint32_t rb = abase + (uint32_t)(wv * 4096 + l8 * 128 + 16 * ((lane & 7) ^ (l8 & 7)));
  const uint64_t wm = uniform_u64_f4(won ? ~0ull : 0ull);
  const uint64_t db = uniform_u64_f4((uint64_t)(a.D + (int64_t)u.row0 * N));
  uint32_t doff = (uint32_t)(l8 * N + ncol0 + 8 * (lane & 7)) * 2u;
  const int dstep = uniform(16 * N);
  const int rbe = uniform(max(2, (u.mrows + 31) / 32));
  const int kb = uniform(KB), mrows = uniform(u.mrows), wons = uniform(won);
  int ks, q, t, inc, inc4, m0v = 0;
  uint64_t sv;
  if constexpr (ROWS == 192)
    MOE_FP4_TALL_ASM(MOE_FP4_TALL192_LOOP_PACKED, MOE_FP4_TALL192_AO_OUTS, MOE_FP4_TALL192_CLOBBERS);
  else
    MOE_FP4_TALL_ASM(MOE_FP4_TALL256_LOOP_PACKED, MOE_FP4_TALL256_AO_OUTS, MOE_FP4_TALL256_CLOBBERS);
}

template <int ROWS>
__global__ __launch_bounds__(256, 1) void gemm_fp4_tall_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t sm[Fp4TallCfg<ROWS>::kLds];
  __shared__ SchedSmem s_sched;
  const Sched sc{&s_sched};
  sched_build<ROWS>(a, sc);
  const Walk walk = sched_walk(s_sched.total);
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  for (int v = walk.first; v < walk.end; v += walk.stride) {
    const Unit u = sched_unit<ROWS>(a, sc, v);
    fp4_unit_tall<ROWS>(a, u, sm, wv, lane);
  }
}

template <int ROWS>
static hipError_t launch_fp4_tall(const GemmArgs& a, hipStream_t s) {
  const int cus = device_info().cus;
  int grid = cus - cus % kXcds;
  if (grid < kXcds) grid = kXcds;
  gemm_fp4_tall_kernel<ROWS><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_fp4(const GemmArgs& a, int expected_m, hipStream_t s) {
  const int em = expected_m > 0 ? expected_m : (a.masked ? a.max_m : 256);
  if (a.wpacked) {
    if (em <= 16) return launch_fp4<1, 3, true>(a, s);  // two K steps in flight per wave (as the FP8 decode tile)
    // the tall tiles copy 4 K blocks of row scales per 16-byte load
    const bool tall_ok = (a.K / 128) % MOE_FP8_TALL_SCALE_GROUP == 0 && (((uintptr_t)a.SFA) & 15) == 0;
    if (em <= 64 || !tall_ok) return launch_fp4<4, 6, true>(a, s);
    if (em >= 256) return launch_fp4_tall<256>(a, s);
    return launch_fp4_tall<192>(a, s);
  }
  if (em <= 16) return launch_fp4<1, 8, false>(a, s);
  return launch_fp4<4, 6, false>(a, s);
}

// ------------------------------------------------------------------ weights --
// E2M1 code of |v| <= 6, round to nearest, ties to the even code; the sign kept (also for a zero result).
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t s = (u >> 28) & 8u;
  const float a = __uint_as_float(u & 0x7fffffffu);
  uint32_t code;
  if (a < 1.0f) {
    code = (uint32_t)__builtin_rintf(a * 2.0f);  // 0, 1 or 2 (code 2 is 1.0); rintf rounds half to even
  } else {
    const uint32_t b = __float_as_uint(a);
    const uint32_t ex = (b >> 23) - 127u;        // 0..2
    const uint32_t keep = (b >> 22) & 1u, rest = b & 0x3fffffu;
    const uint32_t up = (rest > 0x200000u) | ((rest == 0x200000u) & keep);
    code = (ex + 1u) * 2u + keep + up;           // a carry moves to the next binade
  }
  return code | s;
}

// One thread per 32-value block of a weight row: amax, scale 2^e with e the smallest integer such that
// amax <= 6 * 2^e (clamped to [-127, 127], 0 when amax == 0), 16 bytes of codes and the E8M0 byte e + 127.
__global__ __launch_bounds__(256) void quant_weight_fp4_kernel(const uint16_t* __restrict__ w, int64_t nblocks,
                                                               uint8_t* __restrict__ w4, uint8_t* __restrict__ sw) {
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * blockDim.x) {
    float f[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4i raw = *(const v4i*)(w + b * 32 + 8 * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[8 * j + 2 * i] = bf16_to_f32((uint32_t)raw[i] & 0xffffu);
        f[8 * j + 2 * i + 1] = bf16_to_f32((uint32_t)raw[i] >> 16);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
    int e = 0;
    if (amax > 0.0f) {
      // amax = m * 2^x, m in [0.5, 1): 6 * 2^e = 0.75 * 2^(e+3), so e = x - 3 when m <= 0.75, else x - 2
      const int x = __builtin_amdgcn_frexp_expf(amax);
      const float m = __builtin_amdgcn_frexp_mantf(amax);
      e = (m <= 0.75f) ? x - 3 : x - 2;
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    uint32_t out[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= e2m1_encode(__builtin_amdgcn_ldexpf(f[8 * d + i], -e)) << (4 * i);
      out[d] = word;
    }
    *(v4i*)(w4 + b * 16) = v4i{(int)out[0], (int)out[1], (int)out[2], (int)out[3]};
    sw[b] = (uint8_t)(e + 127);
  }
}

// Fragment-packed MXFP4 order (moe_pack_weight_fp4): one thread per 16-byte output chunk of codes, then one
// per output scale dword.  A permutation of bytes; run once when weights are prepared.
__global__ __launch_bounds__(256) void pack_weight_fp4_kernel(const uint8_t* __restrict__ w4, const uint8_t* __restrict__ sw,
                                                              int E, int N, int K, uint8_t* __restrict__ w4p,
                                                              uint8_t* __restrict__ swp) {
  const int ncb = N / 16, n64 = N / 64, kb = K / 128;
  const int64_t cchunks = (int64_t)E * kb * ncb * 64;  // 16-byte code chunks
  const int64_t sdwords = (int64_t)E * kb * n64 * 64;  // scale dwords
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < cchunks + sdwords;
       c += (int64_t)gridDim.x * blockDim.x) {
    if (c < cchunks) {
      // chunk ((e*kb + ks)*ncb + cb)*64 + L: column 16cb + L%16, K 128ks + 32(L/16) .. +31
      const int L = (int)(c & 63);
      int64_t r = c >> 6;
      const int cb = (int)(r % ncb);
      r /= ncb;
      const int ks = (int)(r % kb);
      const int64_t e = r / kb;
      const int64_t n = 16 * cb + (L & 15);
      const v4i v = *(const v4i*)(w4 + (e * N + n) * (K / 2) + 64 * ks + 16 * (L >> 4));
      *(v4i*)(w4p + c * 16) = v;
    } else {
      // dword ((e*kb + ks)*n64 + g64)*64 + L: byte j = scale of column 64 g64 + 16 j + L%16, block 4 ks + L/16
      const int64_t d = c - cchunks;
      const int L = (int)(d & 63);
      int64_t r = d >> 6;
      const int g64 = (int)(r % n64);
      r /= n64;
      const int ks = (int)(r % kb);
      const int64_t e = r / kb;
      const int64_t n0 = 64 * g64 + (L & 15);
      const uint8_t* src = sw + (e * N + n0) * (K / 32) + 4 * ks + (L >> 4);
      const int64_t cs = 16 * (int64_t)(K / 32);  // 16 columns further
      const uint32_t v = (uint32_t)src[0] | ((uint32_t)src[cs] << 8) | ((uint32_t)src[2 * cs] << 16) |
                         ((uint32_t)src[3 * cs] << 24);
      *(uint32_t*)(swp + d * 4) = v;
    }
  }
}

hipError_t launch_pack_weight_fp4(const uint8_t* w4, const uint8_t* sw, int E, int N, int K, uint8_t* w4p,
                                  uint8_t* swp, hipStream_t s) {
  const int64_t work = (int64_t)E * (K / 128) * ((N / 16) * 64 + (N / 64) * 64);
  if (work == 0) return hipSuccess;
  int64_t grid = (work + 255) / 256;
  const int64_t cap = (int64_t)device_info().cus * 8;
  if (grid > cap) grid = cap;
  pack_weight_fp4_kernel<<<(unsigned)grid, 256, 0, s>>>(w4, sw, E, N, K, w4p, swp);
  return hipGetLastError();
}

hipError_t launch_quant_weight_fp4(const uint16_t* w, int E, int N, int K, uint8_t* w4, uint8_t* sw, hipStream_t s) {
  const int64_t nblocks = (int64_t)E * N * (K / 32);
  if (nblocks == 0) return hipSuccess;
  int64_t grid = (nblocks + 255) / 256;
  const int64_t cap = (int64_t)device_info().cus * 16;
  if (grid > cap) grid = cap;
  quant_weight_fp4_kernel<<<(unsigned)grid, 256, 0, s>>>(w, nblocks, w4, sw);
  return hipGetLastError();
}

}  // namespace moe
