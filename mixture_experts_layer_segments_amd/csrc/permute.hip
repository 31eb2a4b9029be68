// Histogram / prefix-sum permutation into contiguous per-expert segments
// ("Serving Mixture-of-Experts Models", section "Follow one token through an
// MoE layer", step 1: a permutation built from a histogram over the expert
// ids, so that the kernels that follow see contiguous per-expert segments).
//
// Four kernels, no global atomics, deterministic output:
//  1. hist:   one block per chunk of assignments counts them per bin
//             (expert, t mod bin_ways) in LDS -> cnt_bin[bin][chunk]; a bin
//             is a replica in the parity split (bin_ways = split_ways), the
//             whole expert otherwise (bin_ways = 1).
//  2. plan:   one block: expert counts, the hot experts, the segment list,
//             seg_offsets (exclusive scan), per-(segment, chunk) bases
//             blk_off[s][b] = seg_offsets[s] + rows of s in chunks < b, and
//             balancedness ("The slowest expert sets the pace").
//  3. rank:   one wave per chunk walks its assignments in order, 64 at a
//             time; lanes of one segment get consecutive rows from their
//             peer mask (one ballot per bit of the segment number), so rows
//             of a segment are in increasing assignment order.
//  4. gather: x_perm[r] = x[row_to_token[r]] with 16-byte loads and stores.
#include "plan_dev.h"
#include "route_dev.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int A,
                                                   int k, int E, int ways, int chunk, int ns,
                                                   int32_t* __restrict__ cnt_bin) {
  __shared__ int h[kMaxBins];
  const int nbins = E * ways;
  for (int i = threadIdx.x; i < nbins; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const int b = blockIdx.x;
  const int a0 = b * chunk;
  const int a1 = min(A, a0 + chunk);
  // four ids per thread loaded before any is counted (one wait on memory
  // per 1024 assignments)
  for (int a = a0 + threadIdx.x; a < a1; a += 4 * 256) {
    int e[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) e[q] = a + 256 * q < a1 ? ids[a + 256 * q] : -1;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (e[q] >= 0 && e[q] < E) atomicAdd(&h[e[q] * ways + ((a + 256 * q) / k) % ways], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nbins; i += blockDim.x) {
    cnt_bin[(size_t)i * ns + b] = h[i];
    // the last chunk's block zeroes the row's padding (chunks nb .. ns-1)
    if (b == (int)gridDim.x - 1)
      for (int j = b + 1; j < ns; ++j) cnt_bin[(size_t)i * ns + j] = 0;
  }
}

// Per-(segment, chunk) bases of the plan: blk_off[s][b] = seg_offsets[s] +
// rows of segment s in chunks < b.  A wave scans a segment's chunk counts,
// lane l taking chunks 4l .. 4l + 3 (rows of the count tables are ns ints,
// nb chunks zero-padded to a multiple of 4), so one wave scan covers the
// segment; wave w takes segments w, w + 16, ...  A chunk count is the
// segment's one bin (a replica of the parity split) or the sum over its
// expert's BW bins.  The loads of QS segments are issued unconditionally,
// from in-range addresses (row 0, the lane's last in-row chunk group) where
// a bin or lane is unused, and masked afterwards: as branches, every load
// waited for its data before the next was issued.  In the load-bounded split
// only the first segment of a hot expert is ever looked up (its rows run on
// through the later ones); the later replica segments get bases too, which
// nothing reads.  Padding segments of the fixed-capacity layout (expert -1)
// get none.  `after_issue` runs once per wave, as soon as the wave's first
// loads are issued (or at once, for a wave without segments): stores issued
// there do not hold up the waits for those loads, which the wave's single
// in-order memory counter would make them do if issued before.
template <int BW, typename F>
__device__ __forceinline__ void segment_bases(const plan_dev::PlanLds& L,
                                              const int32_t* __restrict__ cnt_bin, int S, int nb,
                                              int ns, int32_t* __restrict__ blk_off,
                                              F&& after_issue) {
  constexpr int QS = 16 / BW;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const bool in_row = 4 * lane < nb;
  const int lc = min(lane, ns / 4 - 1);
  bool pending = true;
  for (int sg0 = wv; sg0 < S; sg0 += 16 * QS) {
    int4 u[QS][BW];
    int nbin[QS];
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      const int sg = sg0 + 16 * q;
      const int e = sg < S ? L.seg_exp[sg] : -1;
      int bin0 = 0;
      nbin[q] = 0;
      if (e >= 0) {
        const int f = L.seg_first[e];
        const bool per_replica = BW > 1 && L.seg_first[e + 1] - f > 1;
        bin0 = e * BW + (per_replica ? sg - f : 0);
        nbin[q] = per_replica ? 1 : BW;
      }
      if (!in_row) nbin[q] = 0;
#pragma unroll
      for (int p = 0; p < BW; ++p) {
        const int row = p < nbin[q] ? bin0 + p : 0;
        u[q][p] = reinterpret_cast<const int4*>(cnt_bin + (size_t)row * ns)[lc];
      }
    }
    if (pending) {
      after_issue();
      pending = false;
    }
#pragma unroll
    for (int q = 0; q < QS; ++q) {
      const int sg = sg0 + 16 * q;
      if (sg >= S || L.seg_exp[sg] < 0) continue;
      int4 c = {0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < BW; ++p)
        if (p < nbin[q]) {
          c.x += u[q][p].x;
          c.y += u[q][p].y;
          c.z += u[q][p].z;
          c.w += u[q][p].w;
        }
      const int local = c.x + c.y + c.z + c.w;
      const int incl = plan_dev::wave_incl_scan(local, lane);
      const int r0 = L.seg_off[sg] + incl - local;
      const int4 o = {r0, r0 + c.x, r0 + c.x + c.y, r0 + c.x + c.y + c.z};
      if (in_row) reinterpret_cast<int4*>(blk_off + (size_t)sg * ns)[lane] = o;
    }
  }
  if (pending) after_issue();
}

// WAVE: the one-wave planner (one bin per expert); otherwise the block
// planner with BW bins per expert, or (CAP) the fixed-capacity layout.  Each
// variant holds only the code it runs: one workgroup runs this kernel once,
// and code compiled beside its path, though skipped, measurably slowed it.
template <bool WAVE, int BW, bool CAP>
__global__ __launch_bounds__(1024) void plan_kernel(
    const int32_t* __restrict__ cnt_bin, int nb, int ns, int E, int bin_ways, int ways, int n_hot,
    int c, int cap, int32_t* __restrict__ counts, int32_t* __restrict__ seg_offsets,
    int32_t* __restrict__ seg_expert, int32_t* __restrict__ seg_of_bin,
    int32_t* __restrict__ blk_off, int32_t* __restrict__ r2t, float* __restrict__ bal) {
  __shared__ plan_dev::PlanLds L;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nbins = E * bin_ways;

  // Rows of the count tables are ns ints (nb chunks, zero-padded to a
  // multiple of 4): lane l holds chunks 4l .. 4l + 3 of a row in one 16-byte
  // access (nb <= 256).
  // bin totals: wave w takes bins w, w + 16, ... (QB at a time) and issues
  // all their loads before adding, so it waits on memory once per 16 * QB
  // bins
  constexpr int QB = 16;
  const bool in_row = 4 * lane < nb;
  for (int bin0 = wv; bin0 < nbins; bin0 += 16 * QB) {
    int4 v[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int bin = bin0 + 16 * q;
      v[q] = (bin < nbins && in_row)
                 ? reinterpret_cast<const int4*>(cnt_bin + (size_t)bin * ns)[lane]
                 : int4{0, 0, 0, 0};
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int bin = bin0 + 16 * q;
      const int s = wave_dev::sum(v[q].x + v[q].y + v[q].z + v[q].w);
      if (lane == 0 && bin < nbins) L.tot[bin] = s;
    }
  }
  __syncthreads();
  if constexpr (WAVE) {
    // one segment per expert, planned by one wave; its outputs go out while
    // the bases' loads are in flight
    __shared__ int sob[kMaxE];
    __shared__ float bal_s;
    const int S = plan_dev::plan_segments_by_wave(L, E, sob, &bal_s);
    segment_bases<1>(L, cnt_bin, S, nb, ns, blk_off, [&] {
      plan_dev::write_plan(L, E, counts, seg_offsets, seg_expert, sob, seg_of_bin, bal_s, bal);
    });
  } else {
    int S;
    if constexpr (CAP)
      S = plan_dev::plan_capacity(L, E, cap, counts, seg_offsets, seg_expert, seg_of_bin, r2t,
                                  bal);
    else
      S = plan_dev::plan_segments(L, E, BW, ways, n_hot, c, counts, seg_offsets, seg_expert,
                                  seg_of_bin, bal);
    segment_bases<BW>(L, cnt_bin, S, nb, ns, blk_off, [] {});
  }
}

__global__ __launch_bounds__(64) void rank_kernel(const int32_t* __restrict__ ids, int A, int k,
                                                  int E, int ways, int chunk, int ns, int S,
                                                  int cap,
                                                  const int32_t* __restrict__ seg_of_bin,
                                                  const int32_t* __restrict__ blk_off,
                                                  int32_t* __restrict__ a2r,
                                                  int32_t* __restrict__ r2t,
                                                  const float* __restrict__ w,
                                                  float* __restrict__ row_w) {
  // LDS: run[S], the next free row of each segment; sob[bins], the bin ->
  // segment map
  extern __shared__ int lds[];
  int* run = lds;
  int* sob = lds + S;
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  const int nbins = E * ways;
  const int nbits = plan_dev::segment_bits(S);
  const int a_end = min(A, (b + 1) * chunk);
  // RB rounds of 64 assignments at a time.  The first RB rounds' ids and
  // weights, the chunk's row bases and the bin -> segment map are all loaded
  // before any is used (the loops issue four loads at a time), so the wave
  // waits on memory once before its first round and once per later RB rounds.
  constexpr int RB = 8;
  int e_pre[RB], seg_pre[RB];
  float w_pre[RB];
  const int a_first = b * chunk;
#pragma unroll
  for (int q = 0; q < RB; ++q) {
    const int a = a_first + 64 * q + lane;
    e_pre[q] = a < a_end ? ids[a] : -1;
    w_pre[q] = (row_w && a < a_end) ? w[a] : 0.0f;
  }
#pragma unroll 4
  for (int s = lane; s < S; s += 64) run[s] = blk_off[(size_t)s * ns + b];
#pragma unroll 4
  for (int i = lane; i < nbins; i += 64) sob[i] = seg_of_bin[i];
  __syncthreads();
  for (int a00 = a_first; a00 < a_end; a00 += 64 * RB) {
    if (a00 != a_first) {
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const int a = a00 + 64 * q + lane;
        e_pre[q] = a < a_end ? ids[a] : -1;
        w_pre[q] = (row_w && a < a_end) ? w[a] : 0.0f;
      }
    }
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int a = a00 + 64 * q + lane;
      const int e = e_pre[q];
      seg_pre[q] = (a < a_end && e >= 0 && e < E) ? sob[e * ways + (a / k) % ways] : -1;
    }
    #pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int a0 = a00 + 64 * q;
      if (a0 >= a_end) break;
      const int a = a0 + lane;
      const int seg = seg_pre[q], e = e_pre[q];
      int row = plan_dev::wave_rank_round(seg, nbits, run);
      // fixed capacity: an assignment past its expert's last slot is dropped
      if (cap > 0 && row >= (e + 1) * cap) row = -1;
      if (a < a_end) {
        a2r[a] = row;
        if (row >= 0) {
          r2t[row] = a / k;
          if (row_w) row_w[row] = w_pre[q];
        }
      }
    }
  }
}

// Small batches (decode): routing, histogram, plan and the stable rank in one
// workgroup -- one launch instead of four.  Each wave routes tokens; every
// assignment is binned by LDS atomics (counts do not depend on the order);
// the plan is the one above; and one wave ranks the at most kSmallA
// assignments in order, 64 at a time, as the rank kernel does.
template <int G, int VPL, bool WAVE>
__global__ __launch_bounds__(1024) void route_permute_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int score, int n_group,
    int topk_group, int topn, int renorm, int bin_ways, int ways, int n_hot, int c, int cap,
    int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ counts, int32_t* __restrict__ seg_offsets,
    int32_t* __restrict__ seg_expert, int32_t* __restrict__ a2r, int32_t* __restrict__ r2t,
    float* __restrict__ row_w, float* __restrict__ bal) {
  __shared__ plan_dev::PlanLds L;
  __shared__ int seg_of_bin[kMaxBins];
  __shared__ float bal_s;   // (the one-wave planner's balancedness)
  __shared__ int id_a[kSmallA];
  __shared__ float w_a[kSmallA];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int A = T * k;
  for (int i = tid; i < E * bin_ways; i += 1024) L.tot[i] = 0;
  __syncthreads();
  if constexpr (G > 0) {
    // flat routing on G lanes per token: a wave routes 64 / G tokens at once
    constexpr int TPW = 64 / G;
    const int j = lane % G;
    for (int tb = wv * TPW; tb < T; tb += 16 * TPW) {
      const int t = tb + lane / G;
      float v[VPL];
      route_dev::load_logits_group<G, VPL>(t < T ? logits + (size_t)t * E : nullptr, E, j, v);
      int my_id;
      float my_w;
      route_dev::route_group_vals<G, VPL>(v, E, k, score, renorm, j, my_id, my_w);
      if (t < T && j < k) {
        const int a = t * k + j;
        ids[a] = my_id;
        w[a] = my_w;
        id_a[a] = my_id;
        w_a[a] = my_w;
        atomicAdd(&L.tot[my_id * bin_ways + t % bin_ways], 1);
      }
    }
  }
  // a wave's tokens PF at a time: their logit loads are issued together, so
  // the wave waits on memory once per PF tokens
  // (wide rows, E > 256, keep one token at a time: their registers are taken)
  constexpr int PF = VPL <= 4 ? 4 : 1;
  for (int t0 = wv; G == 0 && t0 < T; t0 += 16 * PF) {
    if constexpr (PF == 1) {
      int my_id;
      float my_w;
      route_dev::route_token<VPL>(logits + (size_t)t0 * E, E, k, score, n_group, topk_group,
                                  topn, renorm, lane, my_id, my_w);
      if (lane < k) {
        const int a = t0 * k + lane;
        ids[a] = my_id;
        w[a] = my_w;
        id_a[a] = my_id;
        w_a[a] = my_w;
        atomicAdd(&L.tot[my_id * bin_ways + t0 % bin_ways], 1);
      }
      continue;
    }
    float v[PF][VPL];
#pragma unroll
    for (int c = 0; c < PF; ++c) {
      const int t = t0 + 16 * c;
      if (t < T) route_dev::load_logits<VPL>(logits + (size_t)t * E, E, lane, v[c]);
    }
#pragma unroll
    for (int c = 0; c < PF; ++c) {
      const int t = t0 + 16 * c;
      if (t >= T) break;
      int my_id;
      float my_w;
      route_dev::route_token_vals<VPL>(v[c], E, k, score, n_group, topk_group, topn, renorm,
                                       lane, my_id, my_w);
      if (lane < k) {
        const int a = t * k + lane;
        ids[a] = my_id;
        w[a] = my_w;
        id_a[a] = my_id;
        w_a[a] = my_w;
        atomicAdd(&L.tot[my_id * bin_ways + t % bin_ways], 1);
      }
    }
  }
  __syncthreads();
  int S;
  if constexpr (WAVE)
    S = plan_dev::plan_segments_by_wave(L, E, seg_of_bin, &bal_s);
  else
    S = cap > 0 ? plan_dev::plan_capacity(L, E, cap, counts, seg_offsets, seg_expert, seg_of_bin,
                                          r2t, bal)
                : plan_dev::plan_segments(L, E, bin_ways, ways, n_hot, c, counts, seg_offsets,
                                          seg_expert, seg_of_bin, bal);
  // the bin totals are spent: L.tot becomes the next free row of each segment
  int* run = L.tot;
  for (int s = tid; s < S; s += 1024) run[s] = L.seg_off[s];
  for (int a = tid; a < A; a += 1024)
    id_a[a] = seg_of_bin[id_a[a] * bin_ways + (a / k) % bin_ways];
  __syncthreads();
  if constexpr (WAVE)
    plan_dev::write_plan(L, E, counts, seg_offsets, seg_expert, seg_of_bin, nullptr, bal_s, bal);
  // one wave ranks every assignment, 64 at a time in assignment order
  if (wv == 0) {
    const int nbits = plan_dev::segment_bits(S);
    for (int a0 = 0; a0 < A; a0 += 64) {
      const int a = a0 + lane;
      const int sa = a < A ? id_a[a] : -1;
      const int row = plan_dev::wave_rank_round(sa, nbits, run);
      if (a >= A) continue;
      if (cap > 0 && row - L.seg_off[sa] >= cap) {   // fixed capacity: the expert's slots are full
        a2r[a] = -1;
        continue;
      }
      a2r[a] = row;
      r2t[row] = a / k;
      row_w[row] = w_a[a];
    }
  }
}

// x_perm[r] = x[row_to_token[r]]: one wave per row, 16-byte chunks.
__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ x,
                                                     const int32_t* __restrict__ r2t,
                                                     const int32_t* __restrict__ total_rows,
                                                     int rows_max, int row_chunks,
                                                     uint4* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows_max || r >= *total_rows) return;
  const int t = r2t[r];
  if (t < 0) return;   // a padding row of the fixed-capacity layout
  const uint4* src = x + (size_t)t * row_chunks;
  uint4* dst = x_perm + (size_t)r * row_chunks;
  int c = lane;
  for (; c + 192 < row_chunks; c += 256) {
    uint4 v0 = src[c], v1 = src[c + 64], v2 = src[c + 128], v3 = src[c + 192];
    dst[c] = v0;
    dst[c + 64] = v1;
    dst[c + 128] = v2;
    dst[c + 192] = v3;
  }
  for (; c < row_chunks; c += 64) dst[c] = src[c];
}

template <int G, int VPL>
void launch_small_vpl(const moe_config& c, const float* logits, int32_t* ids, float* w,
                      int32_t* counts, int32_t* seg_offsets, int32_t* seg_expert, int32_t* a2r,
                      int32_t* r2t, float* row_w, float* bal, hipStream_t s) {
  auto go = [&](auto kernel) {
    kernel<<<1, 1024, 0, s>>>(logits, c.T, c.E, c.k, c.score, c.n_group, c.topk_group,
                              c.group_score_topn, c.renormalize, bin_ways(c), split_ways(c),
                              c.n_hot_split, c.split_c_permille, (int)capacity(c), ids, w,
                              counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal);
  };
  // (the one-wave planner needs E <= 256: only layouts of fewer logits per
  // token than 512 can have it)
  if constexpr ((G > 0 ? G : 64) * VPL < 512) {
    if (wave_plan(c)) return go(route_permute_small_kernel<G, VPL, true>);
  }
  go(route_permute_small_kernel<G, VPL, false>);
}

// Kernel variant for G lanes per token (0: one wave per token) and ceil(E / lanes)
// logits per lane.
template <int G>
void launch_small_g(const moe_config& c, const float* logits, int32_t* ids, float* w,
                    int32_t* counts, int32_t* seg_offsets, int32_t* seg_expert, int32_t* a2r,
                    int32_t* r2t, float* row_w, float* bal, hipStream_t s) {
  const int lanes = G > 0 ? G : 64;
  const int vpl = (c.E + lanes - 1) / lanes;
  if (vpl <= 1)
    launch_small_vpl<G, 1>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
  else if (vpl <= 2)
    launch_small_vpl<G, 2>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
  else if (vpl <= 4)
    launch_small_vpl<G, 4>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
  else if (vpl <= 8)
    launch_small_vpl<G, 8>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
  else
    launch_small_vpl<G, 16>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
}

}  // namespace

void launch_route_permute_small(const moe_config& c, const float* logits, int32_t* ids,
                                float* w, int32_t* counts, int32_t* seg_offsets,
                                int32_t* seg_expert, int32_t* a2r, int32_t* r2t, float* row_w,
                                float* bal, hipStream_t s) {
  const int g = route_dev::flat_group_lanes(c.E, c.k, c.n_group);
  if (g == 16)
    launch_small_g<16>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
  else if (g == 32)
    launch_small_g<32>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
  else
    launch_small_g<0>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
}

void launch_permute(const moe_config& c, const void* x, const int32_t* ids, void* x_perm,
                    int32_t* seg_offsets, int32_t* seg_expert, int32_t* a2r, int32_t* r2t,
                    int32_t* counts, float* bal, const float* w, float* row_w, char* ws,
                    const Layout& L, hipStream_t s) {
  const int A = c.T * c.k;
  const int bw = bin_ways(c);
  const int chunk = chunk_len(A);
  const int nb = num_chunks(A), ns = chunk_stride(A);
  const int S = num_segments(c);
  int32_t* cnt_bin = reinterpret_cast<int32_t*>(ws + L.cnt_bin);
  int32_t* blk_off = reinterpret_cast<int32_t*>(ws + L.blk_off);
  int32_t* seg_of_bin = reinterpret_cast<int32_t*>(ws + L.seg_of_bin);
  hist_kernel<<<nb, 256, 0, s>>>(ids, A, c.k, c.E, bw, chunk, ns, cnt_bin);
  const int cap = (int)capacity(c);
  auto plan = wave_plan(c)      ? plan_kernel<true, 1, false>
              : cap > 0         ? plan_kernel<false, 1, true>
              : bw == 1         ? plan_kernel<false, 1, false>
              : bw == 2         ? plan_kernel<false, 2, false>
              : bw == 3         ? plan_kernel<false, 3, false>
                                : plan_kernel<false, 4, false>;
  plan<<<1, 1024, 0, s>>>(cnt_bin, nb, ns, c.E, bw, split_ways(c), c.n_hot_split,
                          c.split_c_permille, cap, counts, seg_offsets, seg_expert, seg_of_bin,
                          blk_off, r2t, bal);
  // (LDS: the segments' next free rows and the bin -> segment map)
  rank_kernel<<<nb, 64, (size_t)(S + c.E * bw) * sizeof(int), s>>>(
      ids, A, c.k, c.E, bw, chunk, ns, S, cap, seg_of_bin, blk_off, a2r, r2t, w, row_w);
  if (!x_perm) return;  // the caller reads rows of x through row_to_token
  const int eb = c.act_dtype == MOE_DT_F32 ? 4 : 2;
  const int row_chunks = c.H * eb / 16;
  const int R = (int)num_rows(c);
  gather_kernel<<<(R + 3) / 4, 256, 0, s>>>(reinterpret_cast<const uint4*>(x), r2t,
                                            seg_offsets + S, R, row_chunks,
                                            reinterpret_cast<uint4*>(x_perm));
}

}  // namespace moe
