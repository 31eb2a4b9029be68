// Top-k gating kernels: flat routing on 16 or 32 lanes per token, grouped
// routing on one wave64 per token (the per-token logic is in route_dev.h).
#include "route_dev.h"

namespace moe {
namespace {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int score, int n_group,
                                                    int topk_group, int topn, int renorm,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_id;
  float my_w;
  route_dev::route_token<VPL>(logits + (size_t)t * E, E, k, score, n_group, topk_group, topn,
                              renorm, lane, my_id, my_w);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = my_w;
  }
}

// Flat routing, G lanes per token (64 / G tokens per wave, 4 waves per block).
template <int G, int VPL>
__global__ __launch_bounds__(256) void route_group_kernel(const float* __restrict__ logits, int T,
                                                          int E, int k, int score, int renorm,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
  constexpr int TPW = 64 / G;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t0 = (blockIdx.x * 4 + wv) * TPW;
  if (t0 >= T) return;   // the whole wave is past the batch
  const int t = t0 + lane / G, j = lane % G;
  float v[VPL];
  route_dev::load_logits_group<G, VPL>(t < T ? logits + (size_t)t * E : nullptr, E, j, v);
  int my_id;
  float my_w;
  route_dev::route_group_vals<G, VPL>(v, E, k, score, renorm, j, my_id, my_w);
  if (t < T && j < k) {
    ids[(size_t)t * k + j] = my_id;
    w[(size_t)t * k + j] = my_w;
  }
}

template <int G, int VPL>
void launch_group(const moe_config& c, const float* logits, int32_t* ids, float* w,
                  hipStream_t s) {
  const int per_block = 4 * (64 / G);
  route_group_kernel<G, VPL><<<(c.T + per_block - 1) / per_block, 256, 0, s>>>(
      logits, c.T, c.E, c.k, c.score, c.renormalize, ids, w);
}

template <int G>
void launch_group_vpl(const moe_config& c, const float* logits, int32_t* ids, float* w,
                      hipStream_t s) {
  const int vpl = (c.E + G - 1) / G;
  if (vpl <= 1) launch_group<G, 1>(c, logits, ids, w, s);
  else if (vpl <= 2) launch_group<G, 2>(c, logits, ids, w, s);
  else if (vpl <= 4) launch_group<G, 4>(c, logits, ids, w, s);
  else if (vpl <= 8) launch_group<G, 8>(c, logits, ids, w, s);
  else launch_group<G, 16>(c, logits, ids, w, s);
}

template <int VPL>
void launch_vpl(const moe_config& c, const float* logits, int32_t* ids, float* w,
                hipStream_t s) {
  dim3 grid((c.T + 3) / 4);
  route_kernel<VPL><<<grid, 256, 0, s>>>(logits, c.T, c.E, c.k, c.score, c.n_group,
                                          c.topk_group, c.group_score_topn, c.renormalize,
                                          ids, w);
}

}  // namespace

void launch_route(const moe_config& c, const float* logits, int32_t* ids, float* w,
                  hipStream_t s) {
  const int g = route_dev::flat_group_lanes(c.E, c.k, c.n_group);
  if (g == 16) return launch_group_vpl<16>(c, logits, ids, w, s);
  if (g == 32) return launch_group_vpl<32>(c, logits, ids, w, s);
  const int vpl = (c.E + 63) / 64;
  if (vpl <= 1)
    launch_vpl<1>(c, logits, ids, w, s);
  else if (vpl <= 2)
    launch_vpl<2>(c, logits, ids, w, s);
  else if (vpl <= 4)
    launch_vpl<4>(c, logits, ids, w, s);
  else if (vpl <= 8)
    launch_vpl<8>(c, logits, ids, w, s);
  else
    launch_vpl<16>(c, logits, ids, w, s);
}

}  // namespace moe
