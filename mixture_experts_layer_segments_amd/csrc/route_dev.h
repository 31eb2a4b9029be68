// Device-side top-k gating of one token by one wave64 (shared by the routing
// kernel and the fused small-batch routing + permutation kernel).
//
// The token's logits are held in registers (VPL = ceil(E/64) per lane,
// expert e = lane + 64*i) and k rounds of a wave-wide (value desc, id asc)
// arg-max butterfly pick the winners.  Flat mode: the k largest logits;
// weights softmax over the winners.  Grouped mode (the MoE inference blog,
// "MoE architecture recap": a few expert groups first, then the top experts
// inside them): sigmoid scores, each group scored by the fp32 sum of its best
// `topn` member scores, the `topk_group` best groups kept, then the k largest
// logits inside them; weights s_j / sum(s).  Sigmoid and weights are
// evaluated in fp64 and rounded once, so the fp32 group scores (the values
// that decide which groups are kept) are the correctly rounded sigmoid in all
// but vanishingly rare cases.
#pragma once

#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace route_dev {

constexpr int kNoId = 0x7fffffff;

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// Wave-wide arg-max of (value desc, id asc); every lane returns the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(v, off);
    int oi = __shfl_xor(id, off);
    if (better(ov, oi, v, id)) {
      v = ov;
      id = oi;
    }
  }
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Routes the token whose logits start at `row`.  Lane j < k returns slot j:
// its expert id in my_id and its weight (fp64 math rounded once) in my_w.
// This lane's logits of one token row (expert lane + 64 i in slot i, -inf
// past E); the loads of several rows can be issued before any is routed.
template <int VPL>
__device__ __forceinline__ void load_logits(const float* __restrict__ row, int E, int lane,
                                            float (&v)[VPL]) {
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
  }
}

// Routes one token from its loaded logits (load_logits).
template <int VPL>
__device__ __forceinline__ void route_token_vals(const float (&vin)[VPL], int E, int k,
                                                 int score, int n_group, int topk_group,
                                                 int topn, int renorm, int lane,
                                                 int& my_id_out, float& my_w_out) {
  float v[VPL];
  bool avail[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    int e = lane + 64 * i;
    float x = vin[i];
    if (x != x) x = -INFINITY;  // a NaN logit never wins over a number
    v[i] = x;
    avail[i] = e < E;
  }

  if (score == MOE_SCORE_SIGMOID && n_group > 1) {
    const int per = E / n_group;
    float s32[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) s32[i] = (float)(1.0 / (1.0 + exp(-(double)v[i])));
    float my_gs = -INFINITY;  // lane g holds group g's score
    for (int g = 0; g < n_group; ++g) {
      bool used[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i) used[i] = false;
      float acc = 0.0f;
      for (int r = 0; r < topn; ++r) {
        float bv = -INFINITY;
        int bi = kNoId;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          int e = lane + 64 * i;
          if (avail[i] && !used[i] && e / per == g && better(v[i], e, bv, bi)) {
            bv = v[i];
            bi = e;
          }
        }
        wave_argmax(bv, bi);
        if (bi == kNoId) break;  // group smaller than topn
        const int slot = bi >> 6, owner = bi & 63;
        float mine = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (i == slot) mine = s32[i];
        acc = acc + __shfl(mine, owner);
        if (lane == owner) {
#pragma unroll
          for (int i = 0; i < VPL; ++i)
            if (i == slot) used[i] = true;
        }
      }
      if (lane == g) my_gs = acc;
    }
    // keep the topk_group best groups
    uint64_t kept = 0;
    bool gtaken = false;
    for (int r = 0; r < topk_group; ++r) {
      float bv = (lane < n_group && !gtaken) ? my_gs : -INFINITY;
      int bi = (lane < n_group && !gtaken) ? lane : kNoId;
      wave_argmax(bv, bi);
      if (bi == kNoId) break;
      kept |= 1ull << bi;
      if (lane == bi) gtaken = true;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      int e = lane + 64 * i;
      if (avail[i] && !((kept >> (e / per)) & 1ull)) avail[i] = false;
    }
  }

  // k rounds of arg-max over the remaining experts
  int my_id = 0;
  float my_v = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = kNoId;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      int e = lane + 64 * i;
      if (avail[i] && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if (lane == j) {
      my_id = bi;
      my_v = bv;
    }
    if (lane == (bi & 63)) {
      const int slot = bi >> 6;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (i == slot) avail[i] = false;
    }
  }

  // weights in fp64, rounded once
  const double top0 = (double)__shfl(my_v, 0);
  double p = 0.0;
  if (score == MOE_SCORE_SIGMOID) {
    p = lane < k ? 1.0 / (1.0 + exp(-(double)my_v)) : 0.0;
    if (renorm) p = p / wave_sum(p);
  } else {
    p = lane < k ? exp((double)my_v - top0) : 0.0;
    double denom;
    if (renorm) {
      denom = wave_sum(p);
    } else {
      double part = 0.0;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + 64 * i < E) part += exp((double)v[i] - top0);
      denom = wave_sum(part);
    }
    p = p / denom;
  }
  my_id_out = my_id;
  my_w_out = (float)p;
}

// Routes one token whose logit row is `row`.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k,
                                            int score, int n_group, int topk_group, int topn,
                                            int renorm, int lane, int& my_id_out,
                                            float& my_w_out) {
  float v[VPL];
  load_logits<VPL>(row, E, lane, v);
  route_token_vals<VPL>(v, E, k, score, n_group, topk_group, topn, renorm, lane, my_id_out,
                        my_w_out);
}

}  // namespace route_dev
}  // namespace moe
