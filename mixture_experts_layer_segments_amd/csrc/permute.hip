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
//             time; lanes of one segment get consecutive rows from a ballot
//             mask, so rows of a segment are in increasing assignment order.
//  4. gather: x_perm[r] = x[row_to_token[r]] with 16-byte loads and stores.
#include "plan_dev.h"
#include "route_dev.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int A,
                                                   int k, int E, int ways, int chunk, int nb,
                                                   int32_t* __restrict__ cnt_bin) {
  __shared__ int h[kMaxBins];
  const int nbins = E * ways;
  for (int i = threadIdx.x; i < nbins; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const int b = blockIdx.x;
  const int a0 = b * chunk;
  const int a1 = min(A, a0 + chunk);
  for (int a = a0 + threadIdx.x; a < a1; a += blockDim.x) {
    const int e = ids[a];
    if (e >= 0 && e < E) atomicAdd(&h[e * ways + (a / k) % ways], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nbins; i += blockDim.x) cnt_bin[(size_t)i * nb + b] = h[i];
}

__global__ __launch_bounds__(1024) void plan_kernel(
    const int32_t* __restrict__ cnt_bin, int nb, int E, int bin_ways, int ways, int n_hot,
    int c, int cap, int32_t* __restrict__ counts, int32_t* __restrict__ seg_offsets,
    int32_t* __restrict__ seg_expert, int32_t* __restrict__ seg_of_bin,
    int32_t* __restrict__ blk_off, int32_t* __restrict__ r2t, float* __restrict__ bal) {
  __shared__ plan_dev::PlanLds L;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nbins = E * bin_ways;

  // bin totals: a wave takes 4 bins at a time, coalesced over chunks, and
  // issues all their loads (nb <= 256 chunks: 4 per lane and bin) before
  // adding, so it waits on memory once per 4 bins, not once per 64 chunks
  // of every bin
  for (int bin0 = wv; bin0 < nbins; bin0 += 16 * 4) {
    int v[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int bin = bin0 + 16 * q;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int b = lane + 64 * r;
        v[q][r] = (bin < nbins && b < nb) ? cnt_bin[(size_t)bin * nb + b] : 0;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int bin = bin0 + 16 * q;
      int s = v[q][0] + v[q][1] + v[q][2] + v[q][3];
      for (int b = lane + 256; bin < nbins && b < nb; b += 64) s += cnt_bin[(size_t)bin * nb + b];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0 && bin < nbins) L.tot[bin] = s;
    }
  }
  __syncthreads();
  const int S = cap > 0 ? plan_dev::plan_capacity(L, E, cap, counts, seg_offsets, seg_expert,
                                                  seg_of_bin, r2t, bal)
                        : plan_dev::plan_segments(L, E, bin_ways, ways, n_hot, c, counts,
                                                  seg_offsets, seg_expert, seg_of_bin, bal);

  // per-(segment, chunk) bases: a wave scans a segment's chunk counts, lane l
  // taking chunks 4l .. 4l + 3 (nb <= 256), so one wave scan covers the
  // segment.  In the load-bounded split only the first segment of a hot
  // expert is ever looked up (its rows run on through the later ones); the
  // later replica segments get bases too, which nothing reads.  Padding
  // segments of the fixed-capacity layout (expert -1) get none.
  for (int sg = wv; sg < S; sg += 16) {
    const int e = L.seg_exp[sg];
    if (e < 0) continue;
    const int f = L.seg_first[e];
    const bool per_replica = L.seg_first[e + 1] - f > 1 && bin_ways > 1;
    auto count = [&](int b) {
      int v = 0;
      if (b < nb) {
        if (per_replica) {
          v = cnt_bin[(size_t)(e * bin_ways + (sg - f)) * nb + b];
        } else {
          for (int p = 0; p < bin_ways; ++p) v += cnt_bin[(size_t)(e * bin_ways + p) * nb + b];
        }
      }
      return v;
    };
    int v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = count(4 * lane + r);
    const int local = v[0] + v[1] + v[2] + v[3];
    const int incl = plan_dev::wave_incl_scan(local, lane);
    int run = L.seg_off[sg] + incl - local;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int b = 4 * lane + r;
      if (b < nb) blk_off[(size_t)sg * nb + b] = run;
      run += v[r];
    }
  }
}

__global__ __launch_bounds__(64) void rank_kernel(const int32_t* __restrict__ ids, int A, int k,
                                                  int E, int ways, int chunk, int nb, int S,
                                                  int cap,
                                                  const int32_t* __restrict__ seg_of_bin,
                                                  const int32_t* __restrict__ blk_off,
                                                  int32_t* __restrict__ a2r,
                                                  int32_t* __restrict__ r2t,
                                                  const float* __restrict__ w,
                                                  float* __restrict__ row_w) {
  extern __shared__ int run[];  // [S] next free row of each segment
  const int lane = threadIdx.x;
  const int b = blockIdx.x;
  for (int s = lane; s < S; s += 64) run[s] = blk_off[(size_t)s * nb + b];
  __syncthreads();
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int a_end = min(A, (b + 1) * chunk);
  // RB rounds of 64 assignments at a time: their ids, then their segments,
  // are loaded together, so the wave waits on memory twice per RB rounds
  constexpr int RB = 8;
  int e_pre[RB], seg_pre[RB];
  for (int a00 = b * chunk; a00 < a_end; a00 += 64 * RB) {
    #pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int a = a00 + 64 * q + lane;
      e_pre[q] = a < a_end ? ids[a] : -1;
    }
    #pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int a = a00 + 64 * q + lane;
      const int e = e_pre[q];
      seg_pre[q] = (a < a_end && e >= 0 && e < E) ? seg_of_bin[e * ways + (a / k) % ways] : -1;
    }
    #pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int a0 = a00 + 64 * q;
      if (a0 >= a_end) break;
      const int a = a0 + lane;
      const int seg = seg_pre[q], e = e_pre[q];
      int row = -1;
      uint64_t pending = __ballot(seg >= 0);
      while (pending) {
        const int leader = __ffsll((unsigned long long)pending) - 1;
        const int sl = __shfl(seg, leader);
        const uint64_t m = __ballot(seg == sl);
        const int base = run[sl];
        if (seg == sl) row = base + __popcll(m & lt);
        if (lane == leader) run[sl] = base + __popcll(m);
        pending &= ~m;
      }
      // fixed capacity: an assignment past its expert's last slot is dropped
      if (cap > 0 && row >= (e + 1) * cap) row = -1;
      if (a < a_end) {
        a2r[a] = row;
        if (row >= 0) {
          r2t[row] = a / k;
          if (row_w) row_w[row] = w[a];
        }
      }
    }
  }
}

// Small batches (decode): routing, histogram, plan and the stable rank in one
// workgroup -- one launch instead of four.  Each wave routes tokens; every
// assignment is binned by LDS atomics (counts do not depend on the order);
// the plan is the one above; and the row of assignment a is its segment's
// offset plus the number of earlier assignments in the same segment, counted
// directly over the at most kSmallA assignments.
template <int VPL>
__global__ __launch_bounds__(1024) void route_permute_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int score, int n_group,
    int topk_group, int topn, int renorm, int bin_ways, int ways, int n_hot, int c, int cap,
    int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ counts, int32_t* __restrict__ seg_offsets,
    int32_t* __restrict__ seg_expert, int32_t* __restrict__ a2r, int32_t* __restrict__ r2t,
    float* __restrict__ row_w, float* __restrict__ bal) {
  __shared__ plan_dev::PlanLds L;
  __shared__ int seg_of_bin[kMaxBins];
  __shared__ int id_a[kSmallA];
  __shared__ float w_a[kSmallA];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int A = T * k;
  for (int i = tid; i < E * bin_ways; i += 1024) L.tot[i] = 0;
  __syncthreads();
  // a wave's tokens PF at a time: their logit loads are issued together, so
  // the wave waits on memory once per PF tokens
  // (wide rows, E > 256, keep one token at a time: their registers are taken)
  constexpr int PF = VPL <= 4 ? 4 : 1;
  for (int t0 = wv; t0 < T; t0 += 16 * PF) {
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
  if (cap > 0)
    plan_dev::plan_capacity(L, E, cap, counts, seg_offsets, seg_expert, seg_of_bin, r2t, bal);
  else
    plan_dev::plan_segments(L, E, bin_ways, ways, n_hot, c, counts, seg_offsets, seg_expert,
                            seg_of_bin, bal);
  for (int a = tid; a < A; a += 1024)
    id_a[a] = seg_of_bin[id_a[a] * bin_ways + (a / k) % bin_ways];
  __syncthreads();
  for (int a = tid; a < A; a += 1024) {
    const int sa = id_a[a];
    int before = 0;
    for (int b = 0; b < a; ++b) before += id_a[b] == sa;
    if (cap > 0 && before >= cap) {   // fixed capacity: the expert's slots are full
      a2r[a] = -1;
      continue;
    }
    const int row = L.seg_off[sa] + before;
    a2r[a] = row;
    r2t[row] = a / k;
    row_w[row] = w_a[a];
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

template <int VPL>
void launch_small_vpl(const moe_config& c, const float* logits, int32_t* ids, float* w,
                      int32_t* counts, int32_t* seg_offsets, int32_t* seg_expert, int32_t* a2r,
                      int32_t* r2t, float* row_w, float* bal, hipStream_t s) {
  route_permute_small_kernel<VPL><<<1, 1024, 0, s>>>(
      logits, c.T, c.E, c.k, c.score, c.n_group, c.topk_group, c.group_score_topn,
      c.renormalize, bin_ways(c), split_ways(c), c.n_hot_split, c.split_c_permille,
      (int)capacity(c), ids, w, counts, seg_offsets, seg_expert, a2r, r2t,
      row_w, bal);
}

}  // namespace

void launch_route_permute_small(const moe_config& c, const float* logits, int32_t* ids,
                                float* w, int32_t* counts, int32_t* seg_offsets,
                                int32_t* seg_expert, int32_t* a2r, int32_t* r2t, float* row_w,
                                float* bal, hipStream_t s) {
  const int vpl = (c.E + 63) / 64;
  if (vpl <= 1)
    launch_small_vpl<1>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
  else if (vpl <= 2)
    launch_small_vpl<2>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
  else if (vpl <= 4)
    launch_small_vpl<4>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
  else if (vpl <= 8)
    launch_small_vpl<8>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
  else
    launch_small_vpl<16>(c, logits, ids, w, counts, seg_offsets, seg_expert, a2r, r2t, row_w, bal, s);
}

void launch_permute(const moe_config& c, const void* x, const int32_t* ids, void* x_perm,
                    int32_t* seg_offsets, int32_t* seg_expert, int32_t* a2r, int32_t* r2t,
                    int32_t* counts, float* bal, const float* w, float* row_w, char* ws,
                    const Layout& L, hipStream_t s) {
  const int A = c.T * c.k;
  const int bw = bin_ways(c);
  const int chunk = chunk_len(A);
  const int nb = num_chunks(A);
  const int S = num_segments(c);
  int32_t* cnt_bin = reinterpret_cast<int32_t*>(ws + L.cnt_bin);
  int32_t* blk_off = reinterpret_cast<int32_t*>(ws + L.blk_off);
  int32_t* seg_of_bin = reinterpret_cast<int32_t*>(ws + L.seg_of_bin);
  hist_kernel<<<nb, 256, 0, s>>>(ids, A, c.k, c.E, bw, chunk, nb, cnt_bin);
  const int cap = (int)capacity(c);
  plan_kernel<<<1, 1024, 0, s>>>(cnt_bin, nb, c.E, bw, split_ways(c), c.n_hot_split,
                                 c.split_c_permille, cap, counts, seg_offsets, seg_expert,
                                 seg_of_bin, blk_off, r2t, bal);
  rank_kernel<<<nb, 64, S * sizeof(int), s>>>(ids, A, c.k, c.E, bw, chunk, nb, S, cap,
                                              seg_of_bin, blk_off, a2r, r2t, w, row_w);
  if (!x_perm) return;  // the caller reads rows of x through row_to_token
  const int eb = c.act_dtype == MOE_DT_F32 ? 4 : 2;
  const int row_chunks = c.H * eb / 16;
  const int R = (int)num_rows(c);
  gather_kernel<<<(R + 3) / 4, 256, 0, s>>>(reinterpret_cast<const uint4*>(x), r2t,
                                            seg_offsets + S, R, row_chunks,
                                            reinterpret_cast<uint4*>(x_perm));
}

}  // namespace moe
