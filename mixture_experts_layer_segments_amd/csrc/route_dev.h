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
// but vanishingly rare cases.  When a group's experts are an aligned block of
// lanes of one register slot (E / n_group divides 64), all groups are scored
// at once, and only the groups' best members get a sigmoid.
#pragma once

#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace route_dev {

constexpr int kNoId = 0x7fffffff;

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ void take_better(float& v, int& id, float ov, int oi) {
  if (better(ov, oi, v, id)) {
    v = ov;
    id = oi;
  }
}

// One reduction step with the partner lane a DPP row permutation names.
template <int CTRL>
__device__ __forceinline__ void dpp_step(float& v, int& id) {
  const float ov = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, id, CTRL, 0xF, 0xF, false);
  take_better(v, id, ov, oi);
}

// One step with the lane 16 (ROW32 false) or 32 (true) lanes away, by the
// gfx950 row-swap moves: the pair they return holds this lane's own value and
// its partner's, so taking the better of both is the partner step.  (Each
// half of the result is copied into a plain integer before its bit cast:
// bit-casting an element of the builtin's result directly reads element 0.)
template <bool ROW32>
__device__ __forceinline__ void swap_step(float& v, int& id) {
  const uint32_t vb = __builtin_bit_cast(uint32_t, v), ib = (uint32_t)id;
  uint32_t v0, v1, i0, i1;
  if constexpr (ROW32) {
    const auto a = __builtin_amdgcn_permlane32_swap(vb, vb, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(ib, ib, false, false);
    v0 = a[0]; v1 = a[1]; i0 = b[0]; i1 = b[1];
  } else {
    const auto a = __builtin_amdgcn_permlane16_swap(vb, vb, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(ib, ib, false, false);
    v0 = a[0]; v1 = a[1]; i0 = b[0]; i1 = b[1];
  }
  take_better(v, id, __builtin_bit_cast(float, v0), (int)i0);
  take_better(v, id, __builtin_bit_cast(float, v1), (int)i1);
}

// Wave-wide arg-max of (value desc, id asc); every lane returns the winner.
// The partners double the reach each step -- lane l ^ 1, l ^ 2 (quad
// permutations), the mirrored lane of its 8-lane half row and of its 16-lane
// row, then the rows 16 and 32 lanes away -- all register-to-register moves
// (a shuffle by index would go through the LDS unit and wait on it six times
// per arg-max).  The order is total, so the winner is the same whatever the
// reduction order.
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
  dpp_step<0xB1>(v, id);    // quad_perm [1,0,3,2]
  dpp_step<0x4E>(v, id);    // quad_perm [2,3,0,1]
  dpp_step<0x141>(v, id);   // row_half_mirror
  dpp_step<0x140>(v, id);   // row_mirror
  swap_step<false>(v, id);
  swap_step<true>(v, id);
}

// Arg-max of (value desc, id asc) inside every aligned block of P lanes
// (P a power of two up to 64), to every lane of the block: the first log2 P
// steps of wave_argmax.
template <int P>
__device__ __forceinline__ void block_argmax(float& v, int& id) {
  if constexpr (P >= 2) dpp_step<0xB1>(v, id);
  if constexpr (P >= 4) dpp_step<0x4E>(v, id);
  if constexpr (P >= 8) dpp_step<0x141>(v, id);
  if constexpr (P >= 16) dpp_step<0x140>(v, id);
  if constexpr (P >= 32) swap_step<false>(v, id);
  if constexpr (P >= 64) swap_step<true>(v, id);
}

// Group scores when every group of P = E / n_group experts is an aligned
// block of P lanes of one register slot (P divides 64; expert e = lane + 64 i
// sits in slot i): each of the topn rounds takes every group's next best
// member at once, one block arg-max per slot, and lane g (< n_group) adds the
// sigmoid of its group's member -- the group's round-r winner fetched from
// the group's lanes -- to its running score.  The score is the same fp32 sum,
// in the same order of the same correctly rounded fp32 sigmoids, as the
// one-group-at-a-time loop forms; lane g returns group g's score, the others
// -inf.
template <int VPL, int P>
__device__ __forceinline__ float group_scores_blocked(const float (&v)[VPL],
                                                      const bool (&avail)[VPL], int n_group,
                                                      int topn, int lane) {
  bool taken[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) taken[i] = false;
  const int src = (lane * P) & 63, src_slot = (lane * P) >> 6;   // lane g's group
  float acc = 0.0f;
  for (int r = 0; r < topn; ++r) {
    float win = 0.0f;
    bool has = false;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + 64 * i;
      const bool c = avail[i] && !taken[i];
      float bv = c ? v[i] : -INFINITY;
      int bi = c ? e : kNoId;
      block_argmax<P>(bv, bi);
      if (bi == e) taken[i] = true;   // the winner's own lane
      const float wv = __shfl(bv, src);
      const int wi = __shfl(bi, src);
      if (src_slot == i) {
        win = wv;
        has = wi != kNoId;
      }
    }
    if (lane < n_group && has) acc = acc + (float)(1.0 / (1.0 + exp(-(double)win)));
  }
  return lane < n_group ? acc : -INFINITY;
}

// Lane `src` (wave-uniform) of x, to every lane.
__device__ __forceinline__ float lane_value(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src));
}
__device__ __forceinline__ double lane_value(double x, int src) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), src);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum of x over lanes 0 .. n-1 (n wave-uniform, at most 64), in lane order,
// to every lane.
__device__ __forceinline__ double lanes_sum(double x, int n) {
  double s = lane_value(x, 0);
  for (int j = 1; j < n; ++j) s += lane_value(x, j);
  return s;
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
    float my_gs = -INFINITY;  // lane g holds group g's score
    switch (per) {
      case 1: my_gs = group_scores_blocked<VPL, 1>(v, avail, n_group, topn, lane); break;
      case 2: my_gs = group_scores_blocked<VPL, 2>(v, avail, n_group, topn, lane); break;
      case 4: my_gs = group_scores_blocked<VPL, 4>(v, avail, n_group, topn, lane); break;
      case 8: my_gs = group_scores_blocked<VPL, 8>(v, avail, n_group, topn, lane); break;
      case 16: my_gs = group_scores_blocked<VPL, 16>(v, avail, n_group, topn, lane); break;
      case 32: my_gs = group_scores_blocked<VPL, 32>(v, avail, n_group, topn, lane); break;
      case 64: my_gs = group_scores_blocked<VPL, 64>(v, avail, n_group, topn, lane); break;
      default: break;
    }
    // groups that are not lane blocks: one group at a time, over the wave
    float s32[VPL];
    if (64 % per != 0) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) s32[i] = (float)(1.0 / (1.0 + exp(-(double)v[i])));
    }
    for (int g = 0; 64 % per != 0 && g < n_group; ++g) {
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
        bi = __builtin_amdgcn_readfirstlane(bi);   // the same in every lane
        if (bi == kNoId) break;  // group smaller than topn
        const int slot = bi >> 6, owner = bi & 63;
        float mine = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (i == slot) mine = s32[i];
        acc = acc + lane_value(mine, owner);
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
      bi = __builtin_amdgcn_readfirstlane(bi);
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
    bi = __builtin_amdgcn_readfirstlane(bi);
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

  // weights in fp64, rounded once (the winners sit in lanes 0 .. k-1)
  const double top0 = (double)lane_value(my_v, 0);
  double p = 0.0;
  if (score == MOE_SCORE_SIGMOID) {
    p = lane < k ? 1.0 / (1.0 + exp(-(double)my_v)) : 0.0;
    if (renorm) p = p / lanes_sum(p, k);
  } else {
    p = lane < k ? exp((double)my_v - top0) : 0.0;
    double denom;
    if (renorm) {
      denom = lanes_sum(p, k);
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


// ---- flat routing by lane groups ----
// Flat top-k (one expert group) on G = 16 or 32 lanes per token, 64 / G
// tokens per wave: lane j of a group holds experts j + G i (i < VPL), each
// arg-max round reduces inside the group (the first log2 G steps of
// wave_argmax), and the weights of all the wave's tokens are formed together.
// The winners and their order are those of route_token_vals (the order is
// total); the weights' fp64 sum runs in another order (within rounding of the
// same value).

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, true);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// x of the lane 16 lanes away (see swap_step).
__device__ __forceinline__ double swap16_f64(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  const auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const uint32_t l0 = rl[0], l1 = rl[1], h0 = rh[0], h1 = rh[1];
  const bool odd_row = threadIdx.x & 16;
  return __builtin_bit_cast(double, ((uint64_t)(odd_row ? h0 : h1) << 32) | (odd_row ? l0 : l1));
}

template <int G>
__device__ __forceinline__ void group_argmax(float& v, int& id) {
  static_assert(G == 16 || G == 32, "a row or two rows per token");
  dpp_step<0xB1>(v, id);
  dpp_step<0x4E>(v, id);
  dpp_step<0x141>(v, id);
  dpp_step<0x140>(v, id);
  if constexpr (G == 32) swap_step<false>(v, id);
}

template <int G>
__device__ __forceinline__ double group_sum_f64(double x) {
  x += dpp_f64<0xB1>(x);
  x += dpp_f64<0x4E>(x);
  x += dpp_f64<0x141>(x);
  x += dpp_f64<0x140>(x);
  if constexpr (G == 32) x += swap16_f64(x);
  return x;
}

// This lane's logits of the token its group routes (`row`, null past the
// batch: -inf everywhere).
template <int G, int VPL>
__device__ __forceinline__ void load_logits_group(const float* __restrict__ row, int E, int j,
                                                  float (&v)[VPL]) {
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = j + G * i;
    v[i] = (row && e < E) ? row[e] : -INFINITY;
  }
}

// Routes the token of this lane's group from its loaded logits; lane j < k
// of the group returns slot j.
template <int G, int VPL>
__device__ __forceinline__ void route_group_vals(const float (&vin)[VPL], int E, int k, int score,
                                                 int renorm, int j, int& my_id_out,
                                                 float& my_w_out) {
  float v[VPL];
  bool avail[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    float x = vin[i];
    if (x != x) x = -INFINITY;  // a NaN logit never wins over a number
    v[i] = x;
    avail[i] = j + G * i < E;
  }
  int my_id = 0;
  float my_v = 0.0f, top0 = 0.0f;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = kNoId;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = j + G * i;
      if (avail[i] && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
    group_argmax<G>(bv, bi);
    if (r == 0) top0 = bv;
    if (j == r) {
      my_id = bi;
      my_v = bv;
    }
    if (j == bi % G) {
      const int slot = bi / G;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (i == slot) avail[i] = false;
    }
  }
  // weights in fp64, rounded once (the winners sit in lanes 0 .. k-1 of the group)
  double p = 0.0;
  if (score == MOE_SCORE_SIGMOID) {
    p = j < k ? 1.0 / (1.0 + exp(-(double)my_v)) : 0.0;
    if (renorm) p = p / group_sum_f64<G>(p);
  } else {
    p = j < k ? exp((double)my_v - (double)top0) : 0.0;
    double denom;
    if (renorm) {
      denom = group_sum_f64<G>(p);
    } else {
      double part = 0.0;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (j + G * i < E) part += exp((double)v[i] - (double)top0);
      denom = group_sum_f64<G>(part);
    }
    p = p / denom;
  }
  my_id_out = my_id;
  my_w_out = (float)p;
}

// Lanes per token of the flat routing (0: one wave per token, the general
// path): the fewest that hold the k winners, with at most 16 logits per lane.
inline int flat_group_lanes(int E, int k, int n_group) {
  if (n_group > 1) return 0;
  if (k <= 16 && E <= 16 * 16) return 16;
  if (k <= 32 && E <= 16 * 32) return 32;
  return 0;
}

}  // namespace route_dev
}  // namespace moe
