// Top-k gating kernel: one wave64 per token (the per-token logic is in
// route_dev.h).
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
