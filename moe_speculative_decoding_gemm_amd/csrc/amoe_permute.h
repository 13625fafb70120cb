// Group-by-expert of the N*k assignments [MoE-SD blog, MoE layer], as a
// device function run by one work-group of 256 or 1024 threads.
//
// Pass 1 is an LDS histogram (integer atomics: the counts do not depend on
// their order).  One wave scans the counts into offsets while another
// compacts the active experts (and two more, when asked, scan the 64-row
// groups and the cost classes of the work order).  Pass 2 scatters in rounds of 1024 assignments: inside a
// wave, lanes with the same expert find each other with eight ballots over
// the expert-id bits and take their rank from a popcount of the lower peers;
// per-wave totals are scanned across the waves in wave order.  Ranks
// follow assignment order, so the sort is stable and deterministic.
#pragma once

#include "amoe_common.h"

namespace amoe {

struct StatsDev {  // same layout as acceptmoe_stats
  int32_t n_anchor, n_selfsize, n_eligible, n_pruned, n_active, n_active_nonresident,
      n_natural_union, err_flags;
  double r_eff, demand_total;
};

__device__ __forceinline__ int clamp_expert(int e, int E) {
  return e < 0 ? 0 : (e >= E ? E - 1 : e);
}

// exclusive scan of v[0..n) (n <= 256) by one wave; returns the total
__device__ __forceinline__ int wave_exclusive_scan_256(const int* v, int* out, int n) {
  const int lane = lane_id();
  int loc[4];
  int s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = lane * 4 + q;
    loc[q] = s;
    s += idx < n ? v[idx] : 0;
  }
  const int inc = static_cast<int>(wave_inclusive_sum_u32(static_cast<uint32_t>(s)));
  const int base = inc - s;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = lane * 4 + q;
    if (idx < n) out[idx] = base + loc[q];
  }
  return static_cast<int>(readlane_u32(static_cast<uint32_t>(inc), kWave - 1));
}

// LDS of permute_block for NTHR threads
template <int NTHR>
struct PermuteSmem {
  int cnt[kMaxE];
  int off[kMaxE];
  int flag[kMaxE];
  int apos[kMaxE];
  int run[kMaxE];
  int w[NTHR / kWave][kMaxE];
  int wpos[kMaxE];  // position in the work order (active_w)
  int cls[kMaxE];   // cost class flags, packed (see the work order)
  int cpos[kMaxE];  // their exclusive scan
  int ctot;
  int ng[kMaxE];  // 64-row groups of each expert
  int gs[kMaxE];  // their exclusive scan
  int nact, ngrp;
};

// The tables of the grouping from the per-expert counts in sm.cnt[0..E)
// (visible to the whole work-group): offsets, counts, the active list, the
// work order, the row-group table, the largest count and the statistics.
// Leaves the offsets in sm.off for permute_scatter.
template <int NTHR>
__device__ __forceinline__ void permute_tables(int N, int k, int E, int32_t* counts,
                                               int32_t* offsets, int32_t* active,
                                               int32_t* n_active, const uint8_t* resident,
                                               StatsDev* stats, PermuteSmem<NTHR>& sm,
                                               int32_t* max_rows, int32_t* groups,
                                               int32_t* active_w, int group_shift,
                                               int split_rows, int32_t* n_work) {
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = lane_id();
  const int total = N * k;
  // split mode (split_rows >= 0): an expert with more rows is "large"
  const auto large = [&](int c) { return split_rows >= 0 && c > split_rows; };
  if (t < E) {
    const int c = sm.cnt[t];
    sm.flag[t] = c > 0 ? 1 : 0;
    const int ng = (c + (1 << group_shift) - 1) >> group_shift;
    sm.ng[t] = split_rows >= 0 ? (large(c) ? ng : 0) : ng;
    // cost class of the expert's work items (activation rows staged per
    // chunk: 64 / 32 / 16), one 10-bit count field each; none for a large one
    sm.cls[t] = large(c) ? 0 : (c > 32 ? 1 : (c > 16 ? (1 << 10) : (c > 0 ? (1 << 20) : 0)));
  }
  __syncthreads();
  if (wave == 0) {
    wave_exclusive_scan_256(sm.cnt, sm.off, E);
  } else if (wave == 3) {
    const int na = wave_exclusive_scan_256(sm.flag, sm.apos, E);
    if (lane == 0) sm.nact = na;
  } else if (wave == 1 && groups) {
    const int ng = wave_exclusive_scan_256(sm.ng, sm.gs, E);
    if (lane == 0) sm.ngrp = ng;
  } else if (wave == 2 && active_w) {
    const int ct = wave_exclusive_scan_256(sm.cls, sm.cpos, E);
    if (lane == 0) sm.ctot = ct;
  }
  __syncthreads();
  // work order: the active experts by cost class, the class that stages 64
  // rows first, then 32, then 16, each class in index order (in split mode
  // the small experts only, their number in n_work[0]); without active_w it
  // is the active order
  if (t < E) {
    int wp = sm.apos[t];
    if (active_w && sm.flag[t] && !large(sm.cnt[t])) {
      const int c = sm.cnt[t], cp = sm.cpos[t], ct = sm.ctot;
      const int n64 = ct & 1023, n32 = (ct >> 10) & 1023;
      wp = c > 32 ? (cp & 1023) : (c > 16 ? n64 + ((cp >> 10) & 1023) : n64 + n32 + (cp >> 20));
      active_w[wp] = t;
    }
    sm.wpos[t] = wp;
  }
  // the (1 << group_shift)-row groups of the active experts, as
  // (work index << 16 | group), or in split mode the groups of the large
  // experts, as (expert << 16 | group): groups[0] = count, groups[1 + g]
  // = entry g (thread t reads only the work position it wrote)
  if (groups) {
    if (t < E) {
      const int n = sm.ng[t], base = sm.gs[t];
      const int u = split_rows >= 0 ? t : sm.wpos[t];
      for (int j = 0; j < n; ++j) groups[1 + base + j] = (u << 16) | j;
    }
    if (t == 0) groups[0] = sm.ngrp;
  }
  if (n_work && active_w && t == 0) {
    const int ct = sm.ctot;
    n_work[0] = (ct & 1023) + ((ct >> 10) & 1023) + (ct >> 20);
  }
  if (t < E) {
    counts[t] = sm.cnt[t];
    offsets[t] = sm.off[t];
    if (sm.flag[t]) active[sm.apos[t]] = t;
  }
  if (t == 0) {
    offsets[E] = total;
    n_active[0] = sm.nact;
  }
  if (max_rows && t >= kWave && t < 2 * kWave) {  // second wave: the most rows of any expert
    int mr = 0;
    for (int e = t - kWave; e < E; e += kWave) mr = max(mr, sm.cnt[e]);
    mr = static_cast<int>(wave_max_u32(static_cast<uint32_t>(mr)));
    if (t == kWave) max_rows[0] = mr;
  }
  if (stats && t < kWave) {
    int nr = 0;
    if (resident)
      for (int e = t; e < E; e += kWave) nr += (sm.flag[e] && !resident[e]) ? 1 : 0;
    nr = static_cast<int>(readlane_u32(wave_inclusive_sum_u32(static_cast<uint32_t>(nr)), kWave - 1));
    if (t == 0) {
      stats->n_active = sm.nact;
      stats->n_active_nonresident = nr;
    }
  }
}

// Pass 2 of the grouping over the assignments x0 .. x1-1: the first
// assignment of expert e in the range goes to position sm.off[e] +
// sm.run[e] (both set by the caller and visible to the whole work-group);
// advances sm.run.
template <int NTHR>
__device__ __forceinline__ void permute_scatter(int x0, int x1, int E, const int32_t* topk_idx,
                                                int32_t* sorted_assign, int32_t* inv_pos,
                                                PermuteSmem<NTHR>& sm) {
  constexpr int NW = NTHR / kWave;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = lane_id();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = x0; base < x1; base += NTHR) {
    const int x = base + t;
    const bool valid = x < x1;
    const int e = valid ? clamp_expert(topk_idx[x], E) : 0;
    for (int q = lane; q < E; q += kWave) sm.w[wave][q] = 0;
    const uint64_t vmask = __ballot(valid);
    uint64_t peers = vmask;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t mb = __ballot(valid && bit);
      peers &= bit ? mb : ~mb;
    }
    const int rank = __popcll(peers & below);
    if (valid && rank == 0) sm.w[wave][e] = __popcll(peers);
    __syncthreads();
    if (t < E) {
      // only the waves that hold assignments in this round take part
      const int nw = min(NW, (x1 - base + kWave - 1) / kWave);
      int run = sm.run[t];
      for (int w = 0; w < nw; ++w) {
        const int c = sm.w[w][t];
        sm.w[w][t] = run;
        run += c;
      }
      sm.run[t] = run;
    }
    __syncthreads();
    if (valid) {
      const int pos = sm.off[e] + sm.w[wave][e] + rank;
      sorted_assign[pos] = x;
      inv_pos[x] = pos;
    }
    __syncthreads();
  }
}

// Requires blockDim.x == NTHR (256 or 1024).  topk_idx may point to global
// memory or to LDS.  An out-of-range expert id (a caller error) is clamped so
// that no access leaves its buffer.
template <int NTHR>
__device__ __forceinline__ void permute_block(int N, int k, int E, const int32_t* topk_idx,
                                              int32_t* counts, int32_t* offsets,
                                              int32_t* sorted_assign, int32_t* inv_pos,
                                              int32_t* active, int32_t* n_active,
                                              const uint8_t* resident, StatsDev* stats,
                                              PermuteSmem<NTHR>& sm, int32_t* max_rows = nullptr,
                                              int32_t* groups = nullptr,
                                              int32_t* active_w = nullptr,
                                              int group_shift = 6, int split_rows = -1,
                                              int32_t* n_work = nullptr) {
  const int t = threadIdx.x;
  const int total = N * k;
  if (t < kMaxE) {
    sm.cnt[t] = 0;
    sm.run[t] = 0;
  }
  __syncthreads();
  for (int x = t; x < total; x += NTHR) atomicAdd(&sm.cnt[clamp_expert(topk_idx[x], E)], 1);
  __syncthreads();
  permute_tables<NTHR>(N, k, E, counts, offsets, active, n_active, resident, stats, sm, max_rows,
                       groups, active_w, group_shift, split_rows, n_work);
  permute_scatter<NTHR>(0, total, E, topk_idx, sorted_assign, inv_pos, sm);
}

}  // namespace amoe
