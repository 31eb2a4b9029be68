// Register-only collectives of one wave64: DPP row moves and the gfx950 row
// swaps instead of shuffles by lane index, which go through the LDS unit and
// wait on it once per step.  Every lane of the wave must be active.
#pragma once

#include <stdint.h>

namespace moe {
namespace wave_dev {

// x of the lane a DPP control names (0 where it names none, or in rows
// outside ROWS).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, true);
}

// x of the lane 16 (ROW32 false) or 32 (true) lanes away: the row swap
// returns this lane's own value in one half of its result and the partner's
// in the other.  (Each half is copied into a plain integer before use:
// bit-casting an element of the builtin's result directly reads element 0.)
template <bool ROW32>
__device__ __forceinline__ int swap_partner(int x) {
  const uint32_t b = (uint32_t)x;
  uint32_t r0, r1;
  if constexpr (ROW32) {
    const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  return (int)((threadIdx.x & (ROW32 ? 32 : 16)) ? r0 : r1);
}

// Sum of x over the wave, to every lane: partners l ^ 1, l ^ 2 (quad
// permutations), the mirrored lane of the 8-lane half row and of the row,
// then the rows 16 and 32 lanes away.
__device__ __forceinline__ int sum(int x) {
  x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);   // row_half_mirror
  x += dpp<0x140>(x);   // row_mirror
  x += swap_partner<false>(x);
  x += swap_partner<true>(x);
  return x;
}

// The same sum for fp32 values (bit patterns through the same moves).  At
// each step two lanes add the same two partial sums, in either order, and
// fp32 addition commutes: every lane ends with the same bits.
__device__ __forceinline__ float sum(float x) {
  auto step = [](float v, int moved) { return v + __builtin_bit_cast(float, moved); };
  x = step(x, dpp<0xB1>(__builtin_bit_cast(int, x)));
  x = step(x, dpp<0x4E>(__builtin_bit_cast(int, x)));
  x = step(x, dpp<0x141>(__builtin_bit_cast(int, x)));
  x = step(x, dpp<0x140>(__builtin_bit_cast(int, x)));
  x = step(x, swap_partner<false>(__builtin_bit_cast(int, x)));
  x = step(x, swap_partner<true>(__builtin_bit_cast(int, x)));
  return x;
}

// Sum of x over each aligned group of G lanes (G = 1, 2, 4, 8 or 16), to
// every lane of the group: the first log2 G steps of sum().
template <int G>
__device__ __forceinline__ int group_sum(int x) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group of up to one row");
  if constexpr (G >= 2) x += dpp<0xB1>(x);
  if constexpr (G >= 4) x += dpp<0x4E>(x);
  if constexpr (G >= 8) x += dpp<0x141>(x);
  if constexpr (G >= 16) x += dpp<0x140>(x);
  return x;
}

// Maximum of x over the wave, to every lane.
__device__ __forceinline__ int max(int x) {
  x = ::max(x, dpp<0xB1>(x));
  x = ::max(x, dpp<0x4E>(x));
  x = ::max(x, dpp<0x141>(x));
  x = ::max(x, dpp<0x140>(x));
  x = ::max(x, swap_partner<false>(x));
  x = ::max(x, swap_partner<true>(x));
  return x;
}

// Inclusive prefix sum of x over the lanes: shifts by 1, 2, 4 and 8 inside
// each 16-lane row, then the last lane of row 0 (2) added to row 1 (3), then
// lane 31 added to rows 2 and 3.
__device__ __forceinline__ int incl_scan(int x) {
  x += dpp<0x111>(x);         // row_shr:1
  x += dpp<0x112>(x);         // row_shr:2
  x += dpp<0x114>(x);         // row_shr:4
  x += dpp<0x118>(x);         // row_shr:8
  x += dpp<0x142, 0xA>(x);    // row_bcast:15 into rows 1 and 3
  x += dpp<0x143, 0xC>(x);    // row_bcast:31 into rows 2 and 3
  return x;
}

}  // namespace wave_dev
}  // namespace moe
