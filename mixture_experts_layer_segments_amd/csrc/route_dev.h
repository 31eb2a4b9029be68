// Device-side top-k gating of one token by one wave64 (shared by the routing
// kernel and the fused small-batch routing + permutation kernel).
//
// The token's logits are held in registers (VPL = ceil(E/64) per lane,
// expert e = lane + 64*i) and k rounds of a wave-wide (value desc, id asc)
// arg-max butterfly pick the winners; each candidate is one 64-bit key whose
// integer order is that order (sel_key), so a butterfly step is one compare.  Flat mode: the k largest logits;
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

// Selection keys: one 64-bit integer per (value, id) whose unsigned order is
// the routing order -- value descending, then id ascending -- so picking the
// better of two is one integer compare, and the key also carries the value
// and the id.  The high word is the value's bits mapped to an
// order-preserving unsigned integer (+0 and -0 are first made one value, as
// they tie as floats; NaN has already become -inf), so it is at least
// 0x007FFFFF (-inf); the low word is the complement of the id (ids are below
// 2^31).  0 lies below every key and marks a value already taken, a slot past
// the experts or a group not kept.
__device__ __forceinline__ uint64_t sel_key(float x, int id) {
  const uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)id;
}
__device__ __forceinline__ float key_hi_value(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ float key_value(uint64_t key) { return key_hi_value((uint32_t)(key >> 32)); }
__device__ __forceinline__ int key_id(uint64_t key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ uint64_t key_max(uint64_t a, uint64_t b) { return a > b ? a : b; }

// The key of the lane a DPP row permutation names (both words moved).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_key(uint64_t k) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

// The larger of this lane's key and that of the lane 16 (ROW32 false) or 32
// (true) lanes away, by the gfx950 row-swap moves: the pair they return holds
// both.  (Each half of the result is copied into a plain integer before use:
// reading an element of the builtin's result inside a wider expression has
// read element 0.)
template <bool ROW32>
__device__ __forceinline__ uint64_t swap_max_key(uint64_t k) {
  const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  uint32_t l0, l1, h0, h1;
  if constexpr (ROW32) {
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    l0 = a[0]; l1 = a[1]; h0 = b[0]; h1 = b[1];
  } else {
    const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    l0 = a[0]; l1 = a[1]; h0 = b[0]; h1 = b[1];
  }
  return key_max(((uint64_t)h0 << 32) | l0, ((uint64_t)h1 << 32) | l1);
}

// Largest key inside every aligned block of P lanes (P a power of two up to
// 64), to every lane of the block.  The partners double the reach each step
// -- lane l ^ 1, l ^ 2 (quad permutations), the mirrored lane of its 8-lane
// half row and of its 16-lane row, then the rows 16 and 32 lanes away -- all
// register-to-register moves (a shuffle by index would go through the LDS
// unit).  The order is total, so the result does not depend on the order of
// the steps.
template <int P>
__device__ __forceinline__ uint64_t block_max_key(uint64_t k) {
  if constexpr (P >= 2) k = key_max(k, dpp_key<0xB1>(k));    // quad_perm [1,0,3,2]
  if constexpr (P >= 4) k = key_max(k, dpp_key<0x4E>(k));    // quad_perm [2,3,0,1]
  if constexpr (P >= 8) k = key_max(k, dpp_key<0x141>(k));   // row_half_mirror
  if constexpr (P >= 16) k = key_max(k, dpp_key<0x140>(k));  // row_mirror
  if constexpr (P >= 32) k = swap_max_key<false>(k);
  if constexpr (P >= 64) k = swap_max_key<true>(k);
  return k;
}
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) { return block_max_key<64>(k); }

// The same key in every lane, as a wave-uniform (scalar) value.
__device__ __forceinline__ uint64_t uniform_key(uint64_t k) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)k);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(k >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Group scores when every group of P = E / n_group experts is an aligned
// block of P lanes of one register slot (P divides 64; expert e = lane + 64 i
// sits in slot i): each of the topn rounds takes every group's next best
// member at once, one block key maximum per slot, and lane g (< n_group)
// adds the sigmoid of its group's member -- the high word of the group's
// round-r winner, fetched from the group's lanes -- to its running score.
// The score is the same fp32 sum, in the same order of the same correctly
// rounded fp32 sigmoids, as the one-group-at-a-time loop forms; lane g
// returns group g's score, the others -inf.
template <int VPL, int P>
__device__ __forceinline__ float group_scores_blocked(const uint64_t (&key)[VPL], int n_group,
                                                      int topn, int lane) {
  uint64_t kk[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) kk[i] = key[i];
  const int src = (lane * P) & 63, src_slot = (lane * P) >> 6;   // lane g's group
  float acc = 0.0f;
  for (int r = 0; r < topn; ++r) {
    uint32_t win = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const uint64_t best = block_max_key<P>(kk[i]);
      kk[i] = kk[i] == best ? 0 : kk[i];   // the winner's own lane
      const uint32_t w = (uint32_t)__shfl((int)(uint32_t)(best >> 32), src);
      if (src_slot == i) win = w;
    }
    if (lane < n_group && win != 0)
      acc = acc + (float)(1.0 / (1.0 + exp(-(double)key_hi_value(win))));
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
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    float x = vin[i];
    if (x != x) x = -INFINITY;  // a NaN logit never wins over a number
    v[i] = x;
    key[i] = e < E ? sel_key(x, e) : 0;
  }

  if (score == MOE_SCORE_SIGMOID && n_group > 1) {
    const int per = E / n_group;
    float my_gs = -INFINITY;  // lane g holds group g's score
    switch (per) {
      case 1: my_gs = group_scores_blocked<VPL, 1>(key, n_group, topn, lane); break;
      case 2: my_gs = group_scores_blocked<VPL, 2>(key, n_group, topn, lane); break;
      case 4: my_gs = group_scores_blocked<VPL, 4>(key, n_group, topn, lane); break;
      case 8: my_gs = group_scores_blocked<VPL, 8>(key, n_group, topn, lane); break;
      case 16: my_gs = group_scores_blocked<VPL, 16>(key, n_group, topn, lane); break;
      case 32: my_gs = group_scores_blocked<VPL, 32>(key, n_group, topn, lane); break;
      case 64: my_gs = group_scores_blocked<VPL, 64>(key, n_group, topn, lane); break;
      default: break;
    }
    // groups that are not lane blocks: one group at a time, over the wave
    if (64 % per != 0) {
      float s32[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i) s32[i] = (float)(1.0 / (1.0 + exp(-(double)v[i])));
      for (int g = 0; g < n_group; ++g) {
        uint64_t gk[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) gk[i] = (lane + 64 * i) / per == g ? key[i] : 0;
        float acc = 0.0f;
        for (int r = 0; r < topn; ++r) {
          uint64_t best = gk[0];
#pragma unroll
          for (int i = 1; i < VPL; ++i) best = key_max(best, gk[i]);
          best = uniform_key(wave_max_key(best));
          if (best == 0) break;  // group smaller than topn
          const int id = key_id(best);
          const int slot = id >> 6, owner = id & 63;
          float mine = 0.0f;
#pragma unroll
          for (int i = 0; i < VPL; ++i)
            if (i == slot) mine = s32[i];
          acc = acc + lane_value(mine, owner);
#pragma unroll
          for (int i = 0; i < VPL; ++i) gk[i] = gk[i] == best ? 0 : gk[i];
        }
        if (lane == g) my_gs = acc;
      }
    }
    // keep the topk_group best groups (scores ordered like logits: score
    // desc, group id asc)
    uint64_t gkey = lane < n_group ? sel_key(my_gs, lane) : 0;
    uint64_t kept = 0;
    for (int r = 0; r < topk_group; ++r) {
      const uint64_t best = uniform_key(wave_max_key(gkey));
      if (best == 0) break;
      kept |= 1ull << key_id(best);
      gkey = gkey == best ? 0 : gkey;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (!((kept >> ((lane + 64 * i) / per)) & 1ull)) key[i] = 0;
  }

  // k rounds: the wave's largest key is winner j; its lane clears that key
  int my_id = 0;
  float my_v = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = key_max(best, key[i]);
    best = uniform_key(wave_max_key(best));
    if (lane == j) {
      my_id = key_id(best);
      my_v = key_value(best);
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) key[i] = key[i] == best ? 0 : key[i];
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
// arg-max round reduces inside the group (block_max_key<G>), and the weights of all the wave's tokens are formed together.
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
// x of the lane 16 lanes away (the pair the row-swap move returns holds
// this lane's word and its partner's; which is which depends on the row).
__device__ __forceinline__ double swap16_f64(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
  const auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const uint32_t l0 = rl[0], l1 = rl[1], h0 = rh[0], h1 = rh[1];
  const bool odd_row = threadIdx.x & 16;
  return __builtin_bit_cast(double, ((uint64_t)(odd_row ? h0 : h1) << 32) | (odd_row ? l0 : l1));
}

// Largest key over the G lanes of this lane's group (a DPP row, or two).
template <int G>
__device__ __forceinline__ uint64_t group_max_key(uint64_t k) {
  static_assert(G == 16 || G == 32, "a row or two rows per token");
  return block_max_key<G>(k);
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
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    float x = vin[i];
    if (x != x) x = -INFINITY;  // a NaN logit never wins over a number
    v[i] = x;
    key[i] = j + G * i < E ? sel_key(x, j + G * i) : 0;
  }
  // round r: the group's largest key is winner r; its lane clears that key
  int my_id = 0;
  float my_v = 0.0f, top0 = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = key_max(best, key[i]);
    best = group_max_key<G>(best);
    const float bv = key_value(best);
    if (r == 0) top0 = bv;
    if (j == r) {
      my_id = key_id(best);
      my_v = bv;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) key[i] = key[i] == best ? 0 : key[i];
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
