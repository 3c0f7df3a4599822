// route.hip -- moe_route_pack: per-expert counts, segment offsets, a stable
// rank for every route, and the copy of token rows into the packed layout
// (moe_route_pack_quant: the bf16 rows quantised to 1x128 FP8 on the way).
//
// What is computed (rainlin, "GEMM 执行方式", sec. 4.2-4.3, 4.6; AsymGEMM README,
// "Token Layout Protocols"; CuTeDSL bei Perplexity, MoE dispatch):
//   count routes per expert; segment starts = exclusive sum of counts rounded
//   up to the alignment (contiguous) or e*max_m (masked); each route gets a
//   unique index within its expert; rows are copied to start + index.
// The page's scatter allocates rows with an atomic counter, which makes the row
// order within an expert nondeterministic.  Here the index is the route's rank
// among earlier routes to the same expert (route order i = t*k + r), computed
// with wave ballots, so the layout is deterministic and bit-exact.
//
// Launch shapes (the decode/prefill split of CuTeDSL bei Perplexity):
//   R <= 4096 routes: one launch; every workgroup recomputes the routing of all
//     routes in LDS (a few KB) and copies its share of rows -- no grid barrier.
//   R >  4096: three launches -- count (one workgroup per 1024 routes, ranks
//     within the chunk + chunk histogram), scan (one workgroup: per-expert
//     prefix over chunks, segment offsets), gather (bandwidth-sized grid).
#include <mutex>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kDevIdRange = 1, kDevCapacity = 2;
constexpr int kMaxTopk = 64;  // the largest k the C ABI accepts

// Rank of each route among the earlier routes of one 256-route sub-chunk with
// the same expert, plus per-expert totals.  Every thread holds one route id
// (-1 = none).  s_hist[4][E] must be zero on entry and is zero again on exit;
// s_base[e] accumulates the per-expert totals across calls.  Returns the rank
// (base included) for valid ids, -1 otherwise.
__device__ inline int rank_subchunk(int id, int E, int nbits, int* s_hist, int* s_base) {
  const int w = threadIdx.x >> 6;
  const int key = id < 0 ? E : id;
  uint64_t m = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  const int rank_w = __popcll(m & lanemask_lt());
  const int cnt = __popcll(m);
  const bool leader = rank_w == 0;
  if (leader && id >= 0) s_hist[w * kMaxExperts + id] = cnt;
  __syncthreads();
  int rank = -1;
  if (id >= 0) {
    rank = s_base[id] + rank_w;
    for (int w2 = 0; w2 < w; ++w2) rank += s_hist[w2 * kMaxExperts + id];
  }
  __syncthreads();
  if (leader && id >= 0) {
    atomicAdd(&s_base[id], cnt);
    s_hist[w * kMaxExperts + id] = 0;
  }
  __syncthreads();
  return rank;
}

__device__ inline int id_bits(int E) { return 32 - __clz(E); }  // bits to hold 0..E

// Copy one payload row (all lanes of the wave cooperate).  Loads go out in
// batches of 8 per lane before any store: the compiler cannot move a load
// above a store to a possibly aliasing address, so a plain loop would pay one
// memory round trip per 1 KB.  The packed rows are written once and next read
// by the grouped GEMM, so the stores stream past the caches (the whole
// DeepSeek-V3- and Qwen3-shaped steps were 0.3-0.5% faster: no dirty packed
// rows are left to be written back while the GEMM streams its weights).
template <typename T>
__device__ inline void copy_row_as(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t nbytes) {
  constexpr int kB = 8;
  constexpr int64_t kStep = 64 * (int64_t)sizeof(T);
  for (int64_t base = (int64_t)lane_id() * sizeof(T); base < nbytes; base += kB * kStep) {
    T r[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b)
      if (base + b * kStep < nbytes) r[b] = *(const T*)(src + base + b * kStep);
#pragma unroll
    for (int b = 0; b < kB; ++b)
      if (base + b * kStep < nbytes) __builtin_nontemporal_store(r[b], (T*)(dst + base + b * kStep));
  }
}
__device__ inline void copy_row(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t nbytes) {
  const bool v16 = ((nbytes & 15) == 0) && ((((uintptr_t)src) | ((uintptr_t)dst)) & 15) == 0;
  if (v16)
    copy_row_as<v4i>(src, dst, nbytes);
  else
    copy_row_as<uint32_t>(src, dst, nbytes);
}

__device__ inline void place_route(const RouteArgs& a, int i, int p) {
  // p = packed row or -1; all lanes of the wave call this with the same i, p.
  if (lane_id() == 0) a.output_index[i] = p;
  if (p < 0) return;
  const int t = i / a.k;
  copy_row(a.payload + (int64_t)t * a.row_bytes, a.packed + (int64_t)p * a.row_bytes, a.row_bytes);
  if (a.payload2)
    copy_row(a.payload2 + (int64_t)t * a.row_bytes2, a.packed2 + (int64_t)p * a.row_bytes2, a.row_bytes2);
}

// Quantising pack: token t's bf16 row quantised once (1x128 blocks, power-of-
// two scales, E4M3 codes: the rule of moe_quant_act) and written to every
// packed row of its routes, s_p[j] (j < k, -1 = none).  All 4 waves of the
// workgroup call this with the same t: wave w takes the 8-block passes w,
// w + 4, ... (8 lanes per block), so a token's row is spread over the
// workgroup and each lane stores its 16 codes to all k rows.  The block
// scales are collected in s_sc and written as whole scale rows once every
// wave is done (a caller's barrier follows), so each packed scale row is
// one contiguous store rather than eight 32-byte pieces.
__device__ inline void place_token_quant(const RouteArgs& a, int t, const int* s_p, float* s_sc) {
  const int w = threadIdx.x >> 6, lane = lane_id(), sub = lane & 7;
  const int nblk = a.K / 128;
  const uint16_t* x = a.xq + (int64_t)t * a.K;
  for (int b0 = 8 * w; b0 < nblk; b0 += 32) {
    const int blk = b0 + (lane >> 3);
    const bool ok = blk < nblk;
    v4i r0 = {0, 0, 0, 0}, r1 = {0, 0, 0, 0};
    if (ok) {
      r0 = *(const v4i*)(x + (int64_t)blk * 128 + sub * 16);
      r1 = *(const v4i*)(x + (int64_t)blk * 128 + sub * 16 + 8);
    }
    int e;
    const uint4 cw = fp8_block16(r0, r1, e);
    const v4i codes = {(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w};
    if (!ok) continue;
    if (sub == 0) s_sc[blk] = pow2f(e);
    for (int j = 0; j < a.k; ++j) {
      const int p = s_p[j];
      if (p < 0) continue;
      __builtin_nontemporal_store(codes, (v4i*)(a.packed + (int64_t)p * a.K + (int64_t)blk * 128 + sub * 16));
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.k * nblk; i += blockDim.x) {
    const int j = i / nblk, b = i - j * nblk;
    const int p = s_p[j];
    if (p >= 0) __builtin_nontemporal_store(s_sc[b], (float*)a.packed2 + (int64_t)p * nblk + b);
  }
}

// m_indices[r] for r in this workgroup's grid-stride share; s_start[0..E] in LDS.
__device__ inline void fill_m_indices(const RouteArgs& a, const int* s_start) {
  const int64_t total = s_start[a.E];
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < a.rows_cap;
       r += (int64_t)gridDim.x * blockDim.x) {
    int v = -1;
    if (r < total) v = a.masked ? (int)(r / a.max_m) : upper_bound_minus1(s_start, a.E, (int)r);
    a.m_indices[r] = v;
  }
}

// Segment starts from per-expert totals (in s_start[0..E), overwritten).
__device__ inline void segment_starts(const RouteArgs& a, int* s_start, int* s_tmp) {
  if (a.masked) {
    for (int e = threadIdx.x; e <= a.E; e += blockDim.x) s_start[e] = e * a.max_m;
    __syncthreads();
  } else {
    for (int e = threadIdx.x; e < a.E; e += blockDim.x) s_start[e] = (s_start[e] + a.align - 1) / a.align * a.align;
    __syncthreads();
    block_exclusive_scan(s_start, a.E, s_tmp);
  }
}

// ---------------------------------------------------------- single launch --
__global__ __launch_bounds__(256) void route_small_kernel(const RouteArgs a) {
  __shared__ int s_ids[kRouteSmallMax];
  __shared__ int s_rank[kRouteSmallMax];
  __shared__ int s_hist[4 * kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_tmp[257];
  __shared__ int s_flags;
  const int tid = threadIdx.x;
  for (int e = tid; e < 4 * kMaxExperts; e += blockDim.x) s_hist[e] = 0;
  for (int e = tid; e < kMaxExperts; e += blockDim.x) s_base[e] = 0;
  if (tid == 0) s_flags = 0;
  __syncthreads();
  for (int i = tid; i < a.R; i += blockDim.x) {
    int id = a.ids[i];
    if (id >= a.E) {
      atomicOr(&s_flags, kDevIdRange);
      id = -1;
    }
    s_ids[i] = id < 0 ? -1 : id;
  }
  __syncthreads();
  const int nbits = id_bits(a.E);
  for (int c0 = 0; c0 < a.R; c0 += 256) {
    const int i = c0 + tid;
    const int id = i < a.R ? s_ids[i] : -1;
    const int rank = rank_subchunk(id, a.E, nbits, s_hist, s_base);
    if (i < a.R) s_rank[i] = rank;
  }
  // s_base[e] now holds the total routes of expert e
  for (int e = tid; e < a.E; e += blockDim.x) {
    const int tot = s_base[e];
    if (a.masked && tot > a.max_m) atomicOr(&s_flags, kDevCapacity);
    s_start[e] = tot;
  }
  __syncthreads();
  segment_starts(a, s_start, s_tmp);
  if (blockIdx.x == 0) {
    for (int e = tid; e < a.E; e += blockDim.x) a.counts[e] = a.masked ? min(s_base[e], a.max_m) : s_base[e];
    for (int e = tid; e <= a.E; e += blockDim.x) a.seg_offsets[e] = s_start[e];
    if (tid == 0 && s_flags) *a.dev_status |= s_flags;
  }
  const int w = tid >> 6;
  if (a.xq) {
    // quantising pack: one token (its k routes) per workgroup
    __shared__ int s_p[kMaxTopk];
    __shared__ float s_sc[kMaxKBlocks];
    for (int t = blockIdx.x; t < a.T; t += gridDim.x) {
      if (tid < a.k) {
        const int i = t * a.k + tid;
        int p = -1;
        if (s_ids[i] >= 0) {
          const int rank = s_rank[i];
          if (!(a.masked && rank >= a.max_m)) p = s_start[s_ids[i]] + rank;
        }
        a.output_index[i] = p;
        s_p[tid] = p;
      }
      __syncthreads();
      place_token_quant(a, t, s_p, s_sc);
      __syncthreads();  // s_p is rewritten for the next token
    }
  } else {
    for (int i = blockIdx.x * 4 + w; i < a.R; i += gridDim.x * 4) {
      const int id = s_ids[i];
      int p = -1;
      if (id >= 0) {
        const int rank = s_rank[i];
        if (!(a.masked && rank >= a.max_m)) p = s_start[id] + rank;
      }
      place_route(a, i, p);
    }
  }
  fill_m_indices(a, s_start);
}

// ------------------------------------------------------------- large path --
// 1) ranks within a chunk of 1024 routes (kept temporarily in output_index) and
//    the chunk's per-expert histogram.
__global__ __launch_bounds__(256) void route_count_kernel(const RouteArgs a) {
  __shared__ int s_hist[4 * kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_flags;
  const int tid = threadIdx.x;
  for (int e = tid; e < 4 * kMaxExperts; e += blockDim.x) s_hist[e] = 0;
  for (int e = tid; e < kMaxExperts; e += blockDim.x) s_base[e] = 0;
  if (tid == 0) s_flags = 0;
  __syncthreads();
  const int nbits = id_bits(a.E);
  const int c = blockIdx.x;
  // the chunk's ids are loaded up front (one memory round trip, not one per 256-route sub-chunk)
  constexpr int kSubs = kRouteChunk / 256;
  int ids[kSubs];
#pragma unroll
  for (int j = 0; j < kSubs; ++j) {
    const int i = c * kRouteChunk + 256 * j + tid;
    ids[j] = i < a.R ? a.ids[i] : -1;
  }
#pragma unroll
  for (int j = 0; j < kSubs; ++j) {
    const int i = c * kRouteChunk + 256 * j + tid;
    int id = ids[j];
    if (id >= a.E) {
      atomicOr(&s_flags, kDevIdRange);
      id = -1;
    }
    if (id < 0) id = -1;
    const int rank = rank_subchunk(id, a.E, nbits, s_hist, s_base);
    if (i < a.R) a.output_index[i] = rank;
  }
  for (int e = tid; e < a.E; e += blockDim.x) a.ws[(int64_t)c * a.E + e] = s_base[e];
  if (tid == 0) a.ws[(int64_t)a.nchunks * a.E + c] = s_flags;
}

// 2) per-expert prefix over chunks, totals, segment starts, counts, status.
__global__ __launch_bounds__(1024) void route_scan_kernel(const RouteArgs a) {
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_tot[kMaxExperts];
  __shared__ int s_tmp[1025];
  __shared__ int s_flags;
  const int tid = threadIdx.x;
  if (tid == 0) s_flags = 0;
  __syncthreads();
  for (int c = tid; c < a.nchunks; c += blockDim.x) {
    const int f = a.ws[(int64_t)a.nchunks * a.E + c];
    if (f) atomicOr(&s_flags, f);
  }
  for (int e = tid; e < a.E; e += blockDim.x) {
    // 32 chunks' counts are loaded before any prefix is written back (a plain
    // loop would pay one memory round trip per chunk: the store may alias)
    int run = 0;
    for (int c0 = 0; c0 < a.nchunks; c0 += 32) {
      int v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = c0 + j < a.nchunks ? a.ws[(int64_t)(c0 + j) * a.E + e] : 0;
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (c0 + j < a.nchunks) {
          a.ws[(int64_t)(c0 + j) * a.E + e] = run;
          run += v[j];
        }
    }
    s_tot[e] = run;
    s_start[e] = run;
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += blockDim.x)
    if (a.masked && s_tot[e] > a.max_m) atomicOr(&s_flags, kDevCapacity);
  segment_starts(a, s_start, s_tmp);
  for (int e = tid; e < a.E; e += blockDim.x) a.counts[e] = a.masked ? min(s_tot[e], a.max_m) : s_tot[e];
  for (int e = tid; e <= a.E; e += blockDim.x) a.seg_offsets[e] = s_start[e];
  if (tid == 0 && s_flags) *a.dev_status |= s_flags;
}

// 3) final packed row per route, row copies, m_indices.
__global__ __launch_bounds__(256) void route_gather_kernel(const RouteArgs a) {
  __shared__ int s_start[kMaxExperts + 1];
  for (int e = threadIdx.x; e <= a.E; e += blockDim.x) s_start[e] = a.seg_offsets[e];
  __syncthreads();
  const int w = threadIdx.x >> 6;
  auto packed_row = [&](int i) {
    const int id = a.ids[i];
    int p = -1;
    if (id >= 0 && id < a.E) {
      const int local = a.output_index[i];
      const int rank = a.ws[(int64_t)(i / kRouteChunk) * a.E + id] + local;
      if (!(a.masked && rank >= a.max_m)) p = s_start[id] + rank;
    }
    return p;
  };
  if (a.xq) {
    // quantising pack: one token (its k routes) per workgroup; thread j reads route j's rank from output_index
    // and replaces it with the packed row
    __shared__ int s_p[kMaxTopk];
    __shared__ float s_sc[kMaxKBlocks];
    for (int t = blockIdx.x; t < a.T; t += gridDim.x) {
      if (threadIdx.x < a.k) {
        const int i = t * a.k + threadIdx.x;
        const int p = packed_row(i);
        a.output_index[i] = p;
        s_p[threadIdx.x] = p;
      }
      __syncthreads();
      place_token_quant(a, t, s_p, s_sc);
      __syncthreads();  // s_p is rewritten for the next token
    }
  } else {
    for (int i = blockIdx.x * 4 + w; i < a.R; i += gridDim.x * 4) place_route(a, i, packed_row(i));
  }
  fill_m_indices(a, s_start);
}

// Scratch of moe_route_pack_noalloc: the large path's chunk counts and flags
// in a device array of fixed size instead of a caller's workspace.  Host code
// never names the array itself (on the host the name is only a stand-in for
// the symbol): it uses the device address hipGetSymbolAddress returns, looked
// up once per device with that device current.  Every call on one device
// shares the array, so calls that overlap on one device race.  Nothing in it
// needs clearing: the count kernel writes every entry the scan then reads.
constexpr int64_t kRouteScratchBytes = 4ll << 20;
static __device__ __align__(256) int32_t scratch[kRouteScratchBytes / 4];

int64_t route_scratch_bytes() { return kRouteScratchBytes; }

hipError_t route_scratch_ptr(int32_t** out) {
  static std::mutex mu;
  static int32_t* ptrs[kMaxDevices] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = (int32_t*)p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

int64_t route_workspace_bytes(int R, int E) {
  if (R <= kRouteSmallMax) return 0;
  const int64_t nchunks = (R + kRouteChunk - 1) / kRouteChunk;
  return 4 * (nchunks * E + nchunks);
}

hipError_t launch_route_pack(const RouteArgs& a0, hipStream_t s) {
  RouteArgs a = a0;
  const int cus = device_info().cus;
  // one wave per route (quantising: one workgroup per token)
  int gather_grid = a.xq ? a.T : (int)(((int64_t)a.R + 3) / 4);
  const int64_t mi_grid = (a.rows_cap + 255) / 256;
  if (mi_grid > gather_grid) gather_grid = (int)mi_grid;
  if (a.R <= kRouteSmallMax) {
    // every workgroup redoes the routing, so keep the grid near one per CU
    int g = gather_grid < cus ? gather_grid : cus;
    if (g < 1) g = 1;
    a.nchunks = 0;
    route_small_kernel<<<g, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  a.nchunks = (a.R + kRouteChunk - 1) / kRouteChunk;
  route_count_kernel<<<a.nchunks, 256, 0, s>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  route_scan_kernel<<<1, 1024, 0, s>>>(a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  int g = gather_grid < cus * 32 ? gather_grid : cus * 32;
  if (g < 1) g = 1;
  route_gather_kernel<<<g, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
