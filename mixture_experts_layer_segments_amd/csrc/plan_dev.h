// Device-side planning shared by the permutation kernels: block scans and
// the step from bin totals to the segment list ("Serving Mixture-of-Experts
// Models", section "Follow one token through an MoE layer", step 1, and
// section "The slowest expert sets the pace" for balancedness).  Every
// function here is called by all 1024 threads of one workgroup.
#pragma once

#include <type_traits>

#include "moe_internal.h"
#include "wave_dev.h"

namespace moe {
namespace plan_dev {

__device__ __forceinline__ int wave_incl_scan(int v, int) { return wave_dev::incl_scan(v); }

// In-place exclusive scan of n <= 4096 ints in LDS by 1024 threads; returns
// the total to every thread.  The caller has a barrier between its writes of
// data and the call; n <= 64 (a decode batch's experts) is scanned by wave 0
// alone behind one barrier, and then the next call must come after another
// barrier (every thread reads the total from wave_tot).
__device__ inline int block_exclusive_scan(int* data, int n, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (n <= 64) {
    if (wv == 0) {
      const int x = lane < n ? data[lane] : 0;
      const int incl = wave_incl_scan(x, lane);
      if (lane < n) data[lane] = incl - x;
      if (lane == 63) wave_tot[16] = incl;
    }
    __syncthreads();
    return wave_tot[16];
  }
  const int per = (n + 1023) / 1024;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += data[i];
  int incl = wave_incl_scan(sum, lane);
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  if (wv == 0) {
    int x = lane < 16 ? wave_tot[lane] : 0;
    int xi = wave_incl_scan(x, lane);
    if (lane < 16) wave_tot[lane] = xi - x;
    if (lane == 15) wave_tot[16] = xi;
  }
  __syncthreads();
  int run = wave_tot[wv] + incl - sum;
  for (int i = lo; i < hi; ++i) {
    int v = data[i];
    data[i] = run;
    run += v;
  }
  const int total = wave_tot[16];
  __syncthreads();
  return total;
}

// Bits of a segment number below S (0 for S <= 1).
__device__ __forceinline__ int segment_bits(int S) {
  int n = 0;
  while ((1 << n) < S) ++n;
  return n;
}

// Stable rows of one round of 64 assignments (segment `seg` per lane, -1 for
// none) against run[] (LDS, the next free row of each segment): the lanes of
// one segment take consecutive rows in lane order, and run[] of the segment
// advances by their number.  A lane's peers (lanes of its segment) come from
// one ballot per bit of the segment number -- the lanes that agree with it on
// every bit -- so all segments of the round are ranked at once.  Returns the
// row, -1 for seg < 0.  Called by a whole wave.
__device__ __forceinline__ int wave_rank_round(int seg, int nbits, int* run) {
  const int lane = threadIdx.x & 63;
  uint64_t peers = __ballot(seg >= 0);
  for (int j = 0; j < nbits; ++j) {
    const bool bit = (seg >> j) & 1;
    const uint64_t bj = __ballot(bit);
    peers &= bit ? bj : ~bj;
  }
  if (seg < 0) return -1;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int before = __popcll(peers & below);
  const int base = run[seg];
  if (before == 0) run[seg] = base + __popcll(peers);
  return base + before;
}

// LDS scratch of plan_segments, declared by the calling kernel.
struct PlanLds {
  int tot[kMaxBins];            // in: assignments per bin (expert, t mod bin_ways)
  int cnt_e[kMaxE];             // assignments per logical expert
  int seg_first[kMaxE + 1];     // first segment of each expert; [E] = S
  int seg_off[kMaxSegments + 1];  // out: exclusive offsets of the segments
  int seg_exp[kMaxSegments];    // expert of each segment
  int wave_tot[17];
  int red[2][16];
};

// Load of replica p of a hot expert with d assignments in the load-bounded
// split (Zepp paper, section 4.1, Eq. 1 with the integer-rounded bounds and
// the greedy water-filling of section 5, "Routing"): with q = d / ways and
// C = c / 1000 every load lies in [floor(q (1 - C)), ceil(q (1 + C))];
// replicas are filled in order, each up to the upper bound but leaving the
// later replicas their lower bounds.  Exact integer arithmetic.
__device__ inline void bounded_loads(int d, int ways, int c, int* out) {
  const int64_t den = 1000ll * ways;
  const int64_t lb = c >= 1000 ? 0 : (int64_t)d * (1000 - c) / den;
  const int64_t ub = ((int64_t)d * (1000 + c) + den - 1) / den;
  int64_t left = d;
  for (int p = 0; p < ways; ++p) {
    const int64_t n = min(ub, left - (int64_t)(ways - 1 - p) * lb);
    out[p] = (int)n;
    left -= n;
  }
}

// balancedness = (sum/E) / max of the expert counts in L.cnt_e, by one fp64
// division of exact integers ("The slowest expert sets the pace").  Ends with
// a barrier.
__device__ inline void balancedness(PlanLds& L, int E, float* __restrict__ bal) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int mx = 0, sm = 0;
  for (int e = tid; e < E; e += 1024) {
    mx = max(mx, L.cnt_e[e]);
    sm += L.cnt_e[e];
  }
  mx = wave_dev::max(mx);
  sm = wave_dev::sum(sm);
  if (lane == 0) {
    L.red[0][wv] = mx;
    L.red[1][wv] = sm;
  }
  __syncthreads();
  if (tid == 0) {
    int m = 0, su = 0;
    for (int i = 0; i < 16; ++i) {
      m = max(m, L.red[0][i]);
      su += L.red[1][i];
    }
    bal[0] = m > 0 ? (float)(((double)su / (double)E) / (double)m) : 0.0f;
  }
  __syncthreads();
}

// From bin totals to expert counts, the hot experts (the n_hot largest
// counts, lower id on a tie) with `ways` replica segments each, segment
// offsets, the bin -> segment map and balancedness = (sum/E) / max by one fp64
// division of exact integers.  Bins are (expert, t mod bin_ways): bin_ways =
// ways for the parity split (a replica is one bin), 1 otherwise (c >= 0 is
// then the relaxation of the load-bounded split, and every bin maps to the
// expert's first segment: its rows run on through the replica segments).
// Writes counts[E], seg_offsets[S+1], seg_expert[S], seg_of_bin[E*bin_ways]
// and bal[0]; returns S.
__device__ inline int plan_segments(PlanLds& L, int E, int bin_ways, int ways, int n_hot, int c,
                                    int32_t* __restrict__ counts,
                                    int32_t* __restrict__ seg_offsets,
                                    int32_t* __restrict__ seg_expert, int32_t* seg_of_bin,
                                    float* __restrict__ bal) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) {
    int s = 0;
    for (int p = 0; p < bin_ways; ++p) s += L.tot[e * bin_ways + p];
    L.cnt_e[e] = s;
    counts[e] = s;
  }
  __syncthreads();

  const bool split = n_hot > 0 && ways > 1;
  if (split) {
    // rank of each expert among the counts (higher first, lower id on a
    // tie): G adjacent lanes share an expert, each comparing every G-th
    // other expert, and their partial ranks are summed in registers
    auto hot_ranks = [&](auto g_tag) {
      constexpr int G = decltype(g_tag)::value;
      for (int e0 = 0; e0 < E; e0 += 1024 / G) {
        const int e = e0 + tid / G;
        const int ce = e < E ? L.cnt_e[e] : 0;
        int rank = 0;
        if (e < E)
          for (int o = tid % G; o < E; o += G) {
            const int co = L.cnt_e[o];
            rank += (co > ce) || (co == ce && o < e);
          }
        rank = wave_dev::group_sum<G>(rank);
        if (e < E && tid % G == 0) L.seg_first[e] = rank < n_hot ? ways : 1;
      }
    };
    if (E <= 64) hot_ranks(std::integral_constant<int, 16>{});
    else if (E <= 128) hot_ranks(std::integral_constant<int, 8>{});
    else if (E <= 256) hot_ranks(std::integral_constant<int, 4>{});
    else hot_ranks(std::integral_constant<int, 2>{});
  } else {
    for (int e = tid; e < E; e += 1024) L.seg_first[e] = 1;
  }
  __syncthreads();
  const int S = block_exclusive_scan(L.seg_first, E, L.wave_tot);
  if (tid == 0) L.seg_first[E] = S;
  __syncthreads();

  for (int e = tid; e < E; e += 1024) {
    const int f = L.seg_first[e];
    const int nseg = L.seg_first[e + 1] - f;
    for (int p = 0; p < nseg; ++p) {
      L.seg_exp[f + p] = e;
      seg_expert[f + p] = e;
    }
    if (nseg == 1) {
      L.seg_off[f] = L.cnt_e[e];
    } else if (bin_ways > 1) {
      for (int p = 0; p < nseg; ++p) L.seg_off[f + p] = L.tot[e * bin_ways + p];
    } else {
      int loads[kMaxWays];
      bounded_loads(L.cnt_e[e], nseg, c, loads);
      for (int p = 0; p < nseg; ++p) L.seg_off[f + p] = loads[p];
    }
    for (int p = 0; p < bin_ways; ++p) seg_of_bin[e * bin_ways + p] = nseg > 1 ? f + p : f;
  }
  __syncthreads();

  const int total = block_exclusive_scan(L.seg_off, S, L.wave_tot);
  for (int s = tid; s < S; s += 1024) seg_offsets[s] = L.seg_off[s];
  if (tid == 0) {
    seg_offsets[S] = total;
    L.seg_off[S] = total;
  }

  balancedness(L, E, bal);
  return S;
}

// The one-wave planner, for plans that split nothing with E <= 256 (the
// host picks it, wave_plan(); a kernel holds one planner only, since the code
// of the other, run past once by one workgroup, measurably slowed it).  Every
// expert is one segment and one bin (segment e, bin e), so only the row
// offsets need a scan: lane l owns experts l V .. l V + V - 1 (E <= 64 V),
// whose rows are contiguous, and one wave scan of its rows gives them.  The
// results equal plan_segments', without its dozen block barriers (a decode
// batch's plan is latency, not work), and go to LDS only: L, sob (bin ->
// segment) and *bal_s; write_plan() copies them out.  Called by wave 0.
template <int V>
__device__ inline void plan_segments_wave(PlanLds& L, int E, int* sob, float* bal_s) {
  const int lane = threadIdx.x & 63;
  const int e0 = lane * V;
  int cnt[V];
  int cmax = 0, csum = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = e0 + i;
    cnt[i] = e < E ? L.tot[e] : 0;
    cmax = ::max(cmax, cnt[i]);
    csum += cnt[i];
  }
  const int row_incl = wave_dev::incl_scan(csum);
  const int total = __builtin_amdgcn_readlane(row_incl, 63);
  int row = row_incl - csum;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = e0 + i;
    if (e >= E) continue;
    L.cnt_e[e] = cnt[i];
    L.seg_first[e] = e;
    L.seg_exp[e] = e;
    L.seg_off[e] = row;
    sob[e] = e;
    row += cnt[i];
  }
  // balancedness = (sum/E) / max by one fp64 division of exact integers
  const int m = wave_dev::max(cmax);
  if (lane == 0) {
    L.seg_first[E] = E;
    L.seg_off[E] = total;
    *bal_s = m > 0 ? (float)(((double)total / (double)E) / (double)m) : 0.0f;
  }
}

// The one-wave planner by wave 0 of the workgroup; returns S (= E) to every
// thread, after a barrier.
__device__ inline int plan_segments_by_wave(PlanLds& L, int E, int* sob, float* bal_s) {
  if (threadIdx.x < 64) {
    switch ((E + 63) / 64) {
      case 1: plan_segments_wave<1>(L, E, sob, bal_s); break;
      case 2: plan_segments_wave<2>(L, E, sob, bal_s); break;
      case 3: plan_segments_wave<3>(L, E, sob, bal_s); break;
      default: plan_segments_wave<4>(L, E, sob, bal_s); break;
    }
  }
  __syncthreads();
  return E;
}

// The one-wave planner's outputs, by every thread (after a barrier):
// counts[E], seg_offsets[E + 1], seg_expert[E], seg_of_bin[E] (nullable: the
// small kernel keeps the map in LDS) and bal[0].  (A wave's loads and stores
// share one in-order completion counter, so a store issued before a load
// holds up the wait for that load: the callers issue these where no load
// waits behind them.)
__device__ inline void write_plan(const PlanLds& L, int E, int32_t* __restrict__ counts,
                                  int32_t* __restrict__ seg_offsets,
                                  int32_t* __restrict__ seg_expert, const int* sob,
                                  int32_t* __restrict__ seg_of_bin, float bal_s,
                                  float* __restrict__ bal) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) {
    counts[e] = L.cnt_e[e];
    seg_expert[e] = L.seg_exp[e];
    if (seg_of_bin) seg_of_bin[e] = sob[e];
  }
  for (int s = tid; s <= E; s += 1024) seg_offsets[s] = L.seg_off[s];
  if (tid == 0) bal[0] = bal_s;
}

// Fixed-capacity layout (the book's "Capacity, padding, and the drop
// decision"; the MoE inference blog's masked decode layout): expert e owns
// rows [e*cap, (e+1)*cap); segment 2e holds its kept rows (the first
// min(count, cap) of its assignments), segment 2e+1 the unused slots, marked
// with expert -1.  One bin per expert.  Writes counts[E], seg_offsets[2E+1],
// seg_expert[2E], seg_of_bin[E] (-> 2e) and bal[0]; row_to_token = -1 on the
// padding rows; returns S = 2E.  L.seg_first[e] = 2e for the callers.
__device__ inline int plan_capacity(PlanLds& L, int E, int cap, int32_t* __restrict__ counts,
                                    int32_t* __restrict__ seg_offsets,
                                    int32_t* __restrict__ seg_expert, int32_t* seg_of_bin,
                                    int32_t* __restrict__ r2t, float* __restrict__ bal) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) {
    const int c = L.tot[e];
    const int kept = min(c, cap);
    L.cnt_e[e] = c;
    counts[e] = c;
    L.seg_first[e] = 2 * e;
    L.seg_exp[2 * e] = e;
    L.seg_exp[2 * e + 1] = -1;
    L.seg_off[2 * e] = e * cap;
    L.seg_off[2 * e + 1] = e * cap + kept;
    seg_expert[2 * e] = e;
    seg_expert[2 * e + 1] = -1;
    seg_offsets[2 * e] = e * cap;
    seg_offsets[2 * e + 1] = e * cap + kept;
    seg_of_bin[e] = 2 * e;
  }
  if (tid == 0) {
    L.seg_first[E] = 2 * E;
    L.seg_off[2 * E] = E * cap;
    seg_offsets[2 * E] = E * cap;
  }
  __syncthreads();
  const int R = E * cap;
  for (int r = tid; r < R; r += 1024) {
    const int e = r / cap;
    if (r >= L.seg_off[2 * e + 1]) r2t[r] = -1;
  }
  balancedness(L, E, bal);
  return 2 * E;
}

}  // namespace plan_dev
}  // namespace moe
