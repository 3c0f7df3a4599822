// gemm_common.h -- the per-expert tile scheduler shared by the grouped GEMMs.
//
// A unit is (expert e, N-tile of 256 columns, M-chunk of at most BM rows).
// Every workgroup builds the same unit table in LDS from counts (and
// seg_offsets for the contiguous layout) and walks a fixed share of it, so
// there are no atomics and no second launch (AsymGEMM README, "asymScheduler":
// each workgroup owns fixed (N-tile, expert) pairs and reads its rows from the
// offsets table; "K-outer, M-inner Loop": a weight tile is reused by every
// token row of its expert).  Within an expert the units run in 2-D blocks of
// M chunks x N-tiles (sched_unit), so concurrent workgroups that share a
// weight slice or an activation slice find it in the same L2.
//
// XCD awareness: workgroup w runs on XCD w % 8 (round-robin dispatch), so the
// unit list is cut into 8 contiguous slices and the G/8 workgroups of an XCD
// walk their slice in order.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kBN = 256;       // columns per unit (4 waves x 64)
constexpr int kXcds = 8;
constexpr int kNGroup = 8;     // N-tiles per 2-D block of an expert's units

// The unit table in LDS: unit prefix per expert and the expert's rows and first
// packed row, read once from global memory.
struct SchedSmem {
  int up[kMaxExperts + 1];
  int rows[kMaxExperts];
  int start[kMaxExperts];
};
struct Sched {
  SchedSmem* t;
};

// Valid rows and first packed row of expert e (clipped to its segment).
__device__ inline void expert_rows(const GemmArgs& a, int e, int& rows, int& start) {
  int r = a.counts[e];
  int64_t st, cap;
  if (a.masked) {
    st = (int64_t)e * a.max_m;
    cap = a.max_m;
  } else {
    st = a.seg_offsets[e];
    cap = (st >= 0 && st < a.rows_cap) ? a.rows_cap - st : 0;
  }
  if (r < 0) r = 0;
  if (r > cap) r = (int)cap;
  rows = r;
  start = (int)st;
}

// Build the unit table (called by all threads of the workgroup; ends with a
// barrier).  The first wave does the work: each lane takes a run of experts,
// and one wave-wide scan of the lanes' sums gives the prefix -- no barrier
// inside, so the first unit starts about one memory round trip after launch.
template <int BM>
__device__ inline void sched_build(const GemmArgs& a, Sched s) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int nt = (a.N + kBN - 1) / kBN;
    const int per = (a.E + 63) / 64;
    const int e0 = lane * per;
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < a.E) {
        int r, st;
        expert_rows(a, e, r, st);
        s.t->rows[e] = r;
        s.t->start[e] = st;
        s.t->up[e] = sum;  // exclusive within the lane's run
        sum += ((r + BM - 1) / BM) * nt;
      }
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int excl = incl - sum;
    for (int i = 0; i < per; ++i)
      if (e0 + i < a.E) s.t->up[e0 + i] += excl;
    if (lane == 63) s.t->up[a.E] = incl;
  }
  __syncthreads();
}

struct Unit {
  int e, row0, mrows, n0;
};

template <int BM>
__device__ inline Unit sched_unit(const GemmArgs& a, Sched s, int v) {
  const int e = uniform(upper_bound_minus1(s.t->up, a.E, v));
  const int rows = s.t->rows[e], start = s.t->start[e];
  const int local = v - s.t->up[e];
  const int chunks = (rows + BM - 1) / BM;
  // Within an expert the units run in 2-D blocks: groups of kNGroup N-tiles,
  // every M chunk of the group before the next group, the N-tiles of one M
  // chunk adjacent.  A window of 32 consecutive units (one XCD's workgroups)
  // then covers about 4 M chunks x 8 N-tiles: each activation chunk is shared
  // by 8 concurrent units, each weight tile by 4.  (Measured on the
  // Qwen3-shaped GEMMs: groups of 8 beat groups of 16, i.e. the whole width,
  // by 1% on the up-projection and 5% on the down-projection.)
  const int ntiles = (a.N + kBN - 1) / kBN;
  const int full = ntiles / kNGroup;            // complete groups
  const int in_full = full * chunks * kNGroup;  // units in complete groups
  int nt, ch;
  if (local < in_full) {
    const int g = local / (chunks * kNGroup), r = local - g * chunks * kNGroup;
    ch = r / kNGroup;
    nt = g * kNGroup + (r - ch * kNGroup);
  } else {
    const int gl = ntiles - full * kNGroup, r = local - in_full;
    ch = r / gl;
    nt = full * kNGroup + (r - ch * gl);
  }
  Unit u;
  u.e = e;
  u.row0 = uniform(start + ch * BM);
  u.mrows = uniform(min(BM, rows - ch * BM));
  u.n0 = uniform(nt * kBN);
  return u;
}

// This workgroup's slice of the unit list: units lo + slot + i*stride < hi.
struct Walk {
  int first, end, stride;
};
__device__ inline Walk sched_walk(int total_units_any) {
  const int total_units = uniform(total_units_any);
  const int g = gridDim.x;  // a multiple of 8
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, per = g / kXcds;
  const int lo = (int)((int64_t)total_units * xcd / kXcds);
  const int hi = (int)((int64_t)total_units * (xcd + 1) / kXcds);
  Walk w;
  w.first = lo + slot;
  w.end = hi;
  w.stride = per;
  return w;
}

}  // namespace moe
