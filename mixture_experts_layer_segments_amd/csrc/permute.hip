// Histogram / prefix-sum permutation into contiguous per-expert segments
// ("Serving Mixture-of-Experts Models", section "Follow one token through an
// MoE layer", step 1: a permutation built from a histogram over the expert
// ids, so that the kernels that follow see contiguous per-expert segments).
//
// Four kernels, no global atomics, deterministic output:
//  1. hist:   one block per chunk of assignments counts them per bin
//             (expert, t mod ways) in LDS -> cnt_bin[bin][chunk].
//  2. plan:   one block: expert counts, the hot experts, the segment list,
//             seg_offsets (exclusive scan), per-(segment, chunk) bases
//             blk_off[s][b] = seg_offsets[s] + rows of s in chunks < b, and
//             balancedness ("The slowest expert sets the pace").
//  3. rank:   one wave per chunk walks its assignments in order, 64 at a
//             time; lanes of one segment get consecutive rows from a ballot
//             mask, so rows of a segment are in increasing assignment order.
//  4. gather: x_perm[r] = x[row_to_token[r]] with 16-byte loads and stores.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

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

// In-place exclusive scan of n <= 4096 ints in LDS by 1024 threads; returns
// the total to every thread.
__device__ int block_exclusive_scan(int* data, int n, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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

__global__ __launch_bounds__(1024) void plan_kernel(
    const int32_t* __restrict__ cnt_bin, int nb, int E, int ways, int n_hot,
    int32_t* __restrict__ counts, int32_t* __restrict__ seg_offsets,
    int32_t* __restrict__ seg_expert, int32_t* __restrict__ seg_of_bin,
    int32_t* __restrict__ blk_off, float* __restrict__ bal) {
  __shared__ int tot[kMaxBins];
  __shared__ int cnt_e[kMaxE];
  __shared__ int seg_first[kMaxE + 1];
  __shared__ int seg_len[kMaxSegments + 1];
  __shared__ int seg_exp[kMaxSegments];
  __shared__ int wave_tot[17];
  __shared__ int red[2][16];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nbins = E * ways;

  // 1. bin totals: one wave per bin, coalesced over chunks
  for (int bin = wv; bin < nbins; bin += 16) {
    int s = 0;
    for (int b = lane; b < nb; b += 64) s += cnt_bin[(size_t)bin * nb + b];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) tot[bin] = s;
  }
  __syncthreads();

  // 2. logical expert counts
  for (int e = tid; e < E; e += 1024) {
    int s = 0;
    for (int p = 0; p < ways; ++p) s += tot[e * ways + p];
    cnt_e[e] = s;
    counts[e] = s;
  }
  __syncthreads();

  // 3. hot experts: rank by (count desc, id asc); segments per expert
  const bool split = n_hot > 0 && ways > 1;
  for (int e = tid; e < E; e += 1024) {
    int nseg = 1;
    if (split) {
      const int ce = cnt_e[e];
      int rank = 0;
      for (int o = 0; o < E; ++o) {
        const int co = cnt_e[o];
        rank += (co > ce) || (co == ce && o < e);
      }
      if (rank < n_hot) nseg = ways;
    }
    seg_first[e] = nseg;
  }
  __syncthreads();
  const int S = block_exclusive_scan(seg_first, E, wave_tot);
  if (tid == 0) seg_first[E] = S;
  __syncthreads();

  // 4. segment list, lengths, bin -> segment map
  for (int e = tid; e < E; e += 1024) {
    const int f = seg_first[e];
    const int nseg = seg_first[e + 1] - f;
    for (int p = 0; p < nseg; ++p) {
      seg_exp[f + p] = e;
      seg_expert[f + p] = e;
      seg_len[f + p] = nseg > 1 ? tot[e * ways + p] : cnt_e[e];
    }
    for (int p = 0; p < ways; ++p) seg_of_bin[e * ways + p] = nseg > 1 ? f + p : f;
  }
  __syncthreads();

  // 5. segment offsets
  const int total = block_exclusive_scan(seg_len, S, wave_tot);
  for (int s = tid; s < S; s += 1024) seg_offsets[s] = seg_len[s];
  if (tid == 0) seg_offsets[S] = total;

  // 6. per-(segment, chunk) bases: one wave per segment scans over chunks
  for (int s = wv; s < S; s += 16) {
    const int e = seg_exp[s];
    const int f = seg_first[e];
    const bool hot = seg_first[e + 1] - f > 1;
    int carry = seg_len[s];
    for (int b0 = 0; b0 < nb; b0 += 64) {
      const int b = b0 + lane;
      int v = 0;
      if (b < nb) {
        if (hot) {
          v = cnt_bin[(size_t)(e * ways + (s - f)) * nb + b];
        } else {
          for (int p = 0; p < ways; ++p) v += cnt_bin[(size_t)(e * ways + p) * nb + b];
        }
      }
      const int incl = wave_incl_scan(v, lane);
      if (b < nb) blk_off[(size_t)s * nb + b] = carry + incl - v;
      carry += __shfl(incl, 63);
    }
  }

  // 7. balancedness = (sum / E) / max, one fp64 division of exact integers
  int mx = 0, sm = 0;
  for (int e = tid; e < E; e += 1024) {
    mx = max(mx, cnt_e[e]);
    sm += cnt_e[e];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mx = max(mx, __shfl_xor(mx, off));
    sm += __shfl_xor(sm, off);
  }
  if (lane == 0) {
    red[0][wv] = mx;
    red[1][wv] = sm;
  }
  __syncthreads();
  if (tid == 0) {
    int m = 0, su = 0;
    for (int i = 0; i < 16; ++i) {
      m = max(m, red[0][i]);
      su += red[1][i];
    }
    bal[0] = m > 0 ? (float)(((double)su / (double)E) / (double)m) : 0.0f;
  }
}

__global__ __launch_bounds__(64) void rank_kernel(const int32_t* __restrict__ ids, int A, int k,
                                                  int E, int ways, int chunk, int nb, int S,
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
  for (int a0 = b * chunk; a0 < a_end; a0 += 64) {
    const int a = a0 + lane;
    int seg = -1;
    if (a < a_end) {
      const int e = ids[a];
      if (e >= 0 && e < E) seg = seg_of_bin[e * ways + (a / k) % ways];
    }
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
    if (a < a_end) {
      a2r[a] = row;
      if (row >= 0) {
        r2t[row] = a / k;
        if (row_w) row_w[row] = w[a];
      }
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

}  // namespace

void launch_permute(const moe_config& c, const void* x, const int32_t* ids, void* x_perm,
                    int32_t* seg_offsets, int32_t* seg_expert, int32_t* a2r, int32_t* r2t,
                    int32_t* counts, float* bal, const float* w, float* row_w, char* ws,
                    const Layout& L, hipStream_t s) {
  const int A = c.T * c.k;
  const int ways = c.n_hot_split > 0 ? c.split_ways : 1;
  const int chunk = chunk_len(A);
  const int nb = num_chunks(A);
  const int S = num_segments(c);
  int32_t* cnt_bin = reinterpret_cast<int32_t*>(ws + L.cnt_bin);
  int32_t* blk_off = reinterpret_cast<int32_t*>(ws + L.blk_off);
  int32_t* seg_of_bin = reinterpret_cast<int32_t*>(ws + L.seg_of_bin);
  hist_kernel<<<nb, 256, 0, s>>>(ids, A, c.k, c.E, ways, chunk, nb, cnt_bin);
  plan_kernel<<<1, 1024, 0, s>>>(cnt_bin, nb, c.E, ways, c.n_hot_split, counts, seg_offsets,
                                 seg_expert, seg_of_bin, blk_off, bal);
  rank_kernel<<<nb, 64, S * sizeof(int), s>>>(ids, A, c.k, c.E, ways, chunk, nb, S,
                                              seg_of_bin, blk_off, a2r, r2t, w, row_w);
  if (!x_perm) return;  // the caller reads rows of x through row_to_token
  const int eb = c.act_dtype == MOE_DT_F32 ? 4 : 2;
  const int row_chunks = c.H * eb / 16;
  gather_kernel<<<(A + 3) / 4, 256, 0, s>>>(reinterpret_cast<const uint4*>(x), r2t,
                                            seg_offsets + S, A, row_chunks,
                                            reinterpret_cast<uint4*>(x_perm));
}

}  // namespace moe
