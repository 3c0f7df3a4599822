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
// Balance: the list is sorted by cost (full chunks, then partial chunks by
// size) and dealt in rounds of one unit per workgroup, so the units of a
// round cost about the same and no workgroup collects the expensive ones.
// XCD awareness: workgroup w runs on XCD w % 8 (round-robin dispatch), so a
// round goes to the G/8 workgroups of one XCD (sched_walk).
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kBN = 256;       // columns per unit (4 waves x 64)
constexpr int kXcds = 8;
constexpr int kNGroup = 8;     // N-tiles per 2-D block of an expert's units

// The unit table in LDS.  Units are ordered by cost, so that the workgroups
// dealt one round of units at a time finish together: first every full chunk
// (BM rows) of every expert, then the experts' last, partial chunks, largest
// first (ties by expert).  The rows of a partial chunk are counted in steps
// of the tile heights' row granularity.
struct SchedSmem {
  int up[kMaxExperts + 1];  // full-chunk units before expert e; up[E] = all of them
  int tail_e[kMaxExperts];  // expert of the q-th partial chunk in cost order
  int rows[kMaxExperts];
  int start[kMaxExperts];
  int total;                // all units
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

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Build the unit table (called by all threads of the workgroup; ends with a
// barrier).  The first wave does the work: each lane takes a run of experts;
// a wave-wide scan gives the full-chunk prefix, and one scan per size class
// of the partial chunks gives their places (a counting sort).
template <int BM>
__device__ inline void sched_build(const GemmArgs& a, Sched s) {
  constexpr int kGran = BM >= 128 ? 32 : 16;  // rows per tile-height step
  constexpr int kCls = (BM + kGran - 1) / kGran;
  static_assert(kCls <= 15, "size class in 4 bits");
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int nt = (a.N + kBN - 1) / kBN;
    const int per = (a.E + 63) / 64;  // <= 16
    const int e0 = lane * per;
    int sum = 0;
    uint64_t cls = 0;  // size class of each of the lane's experts' partial chunk (0: none), 4 bits each
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < a.E) {
        int r, st;
        expert_rows(a, e, r, st);
        s.t->rows[e] = r;
        s.t->start[e] = st;
        s.t->up[e] = sum;  // exclusive within the lane's run
        sum += (r / BM) * nt;
        cls |= (uint64_t)((r % BM + kGran - 1) / kGran) << (4 * i);
      }
    }
    const int incl = wave_incl_scan(sum, lane);
    const int excl = incl - sum;
    for (int i = 0; i < per; ++i)
      if (e0 + i < a.E) s.t->up[e0 + i] += excl;
    const int ufull = __shfl(incl, 63, 64);
    if (lane == 63) s.t->up[a.E] = incl;
    int base = 0;
    for (int c = kCls; c >= 1; --c) {
      int cnt = 0;
      for (int i = 0; i < per; ++i) cnt += ((cls >> (4 * i)) & 15) == (uint64_t)c;
      const int ci = wave_incl_scan(cnt, lane);
      int pos = base + ci - cnt;
      for (int i = 0; i < per; ++i)
        if (((cls >> (4 * i)) & 15) == (uint64_t)c) s.t->tail_e[pos++] = e0 + i;
      base += __shfl(ci, 63, 64);
    }
    if (lane == 0) s.t->total = ufull + base * nt;
  }
  __syncthreads();
}

struct Unit {
  int e, row0, mrows, n0;
};

template <int BM>
__device__ inline Unit sched_unit(const GemmArgs& a, Sched s, int v) {
  const int ntiles = (a.N + kBN - 1) / kBN;
  const int ufull = s.t->up[a.E];
  int e, ch, nt;
  if (v < ufull) {
    e = uniform(upper_bound_minus1(s.t->up, a.E, v));
    const int local = v - s.t->up[e];
    const int chunks = s.t->rows[e] / BM;
    // The full chunks of an expert run in 2-D blocks: groups of kNGroup
    // N-tiles, every chunk of the group before the next group, the N-tiles of
    // one chunk adjacent.  A round of 32 consecutive units (one XCD's
    // workgroups) then covers about 4 chunks x 8 N-tiles: each activation
    // chunk is shared by 8 concurrent units, each weight tile by 4.
    const int full = ntiles / kNGroup;            // complete groups
    const int in_full = full * chunks * kNGroup;  // units in complete groups
    if (local < in_full) {
      const int g = local / (chunks * kNGroup), r = local - g * chunks * kNGroup;
      ch = r / kNGroup;
      nt = g * kNGroup + (r - ch * kNGroup);
    } else {
      const int gl = ntiles - full * kNGroup, r = local - in_full;
      ch = r / gl;
      nt = full * kNGroup + (r - ch * gl);
    }
  } else {
    // partial chunks: the N-tiles of one chunk adjacent
    const int w = v - ufull, q = w / ntiles;
    nt = w - q * ntiles;
    e = uniform(s.t->tail_e[q]);
    ch = s.t->rows[e] / BM;
  }
  const int rows = s.t->rows[e], start = s.t->start[e];
  Unit u;
  u.e = e;
  u.row0 = uniform(start + ch * BM);
  u.mrows = uniform(min(BM, rows - ch * BM));
  u.n0 = uniform(nt * kBN);
  return u;
}

// This workgroup's units: first, first + stride, ... < end.  The unit list is
// dealt in rounds of G/8 consecutive units, round r to XCD r mod 8
// (workgroup w runs on XCD w mod 8), one unit per workgroup of that XCD: the
// units of a round share weights or activations in that XCD's L2, and the 8
// rounds in flight at once are neighbours in the list (the same expert's
// weights for a large expert), which the shared last-level cache serves.
struct Walk {
  int first, end, stride;
};
__device__ inline Walk sched_walk(int total_units_any) {
  const int total_units = uniform(total_units_any);
  const int g = gridDim.x;  // a multiple of 8
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, per = g / kXcds;
  Walk w;
  w.first = per * xcd + slot;
  w.end = total_units;
  w.stride = g;
  return w;
}

}  // namespace moe
