// Inverse permutation with a router-weighted sum ("Serving Mixture-of-Experts
// Models", section "Follow one token through an MoE layer", step 4):
// out[t] = sum_j w[t,j] * y_perm[assign_to_row[t*k+j]] (+ shared_y[t]).
// One thread per 16-byte chunk of an output row: it accumulates the chunk of
// the token's k rows in fp32 in slot order and rounds once.  No atomics.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint4 pack_bf16x8(const float* f) {
  uint4 u;
  u.x = bf16_bits_rne(f[0]) | (bf16_bits_rne(f[1]) << 16);
  u.y = bf16_bits_rne(f[2]) | (bf16_bits_rne(f[3]) << 16);
  u.z = bf16_bits_rne(f[4]) | (bf16_bits_rne(f[5]) << 16);
  u.w = bf16_bits_rne(f[6]) | (bf16_bits_rne(f[7]) << 16);
  return u;
}

// y_perm rows are read once and out is written once, so both go through
// non-temporal accesses, and each thread issues the loads of 4 rows at a
// time.  Measured: the layer 0.4-3% faster across the workloads (most on the
// prefill and ragged ones), bit-identical outputs.
constexpr int kCombineRows = 4;   // y rows loaded together per output chunk

// A 16-byte chunk of a y_perm row.
__device__ __forceinline__ uint4 load_row_chunk(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y,
                                                      const int32_t* __restrict__ a2r,
                                                      const float* __restrict__ w,
                                                      const uint4* __restrict__ shared_y,
                                                      int T, int k, int row_chunks,
                                                      uint4* __restrict__ out) {
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * row_chunks) return;
  const int t = (int)(idx / row_chunks);
  const int c = (int)(idx % row_chunks);
  const int32_t* rows = a2r + (size_t)t * k;
  const float* wt = w ? w + (size_t)t * k : nullptr;
  {
    float acc[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) acc[i] = 0.0f;
    // CU rows at a time: their loads are issued together, then summed in
    // slot order (the same fp32 operations in the same order as one by one)
    for (int j0 = 0; j0 < k; j0 += kCombineRows) {
      uint4 u[kCombineRows];
      float wj[kCombineRows];
      bool ok[kCombineRows];
#pragma unroll
      for (int q = 0; q < kCombineRows; ++q) {
        const int j = j0 + q;
        const int r = j < k ? rows[j] : -1;
        ok[q] = r >= 0;
        wj[q] = (ok[q] && wt) ? wt[j] : 1.0f;
        u[q] = ok[q] ? load_row_chunk(y + (size_t)r * row_chunks + c) : uint4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < kCombineRows; ++q) {
        if (!ok[q]) continue;
        float f[EPC];
        if constexpr (BF16) {
          unpack_bf16x8(u[q], f);
        } else {
          f[0] = __uint_as_float(u[q].x);
          f[1] = __uint_as_float(u[q].y);
          f[2] = __uint_as_float(u[q].z);
          f[3] = __uint_as_float(u[q].w);
        }
#pragma unroll
        for (int i = 0; i < EPC; ++i) acc[i] = fmaf(wj[q], f[i], acc[i]);
      }
    }
    if (shared_y) {
      const uint4 u = shared_y[(size_t)t * row_chunks + c];
      float f[EPC];
      if constexpr (BF16) {
        unpack_bf16x8(u, f);
      } else {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
      }
#pragma unroll
      for (int i = 0; i < EPC; ++i) acc[i] += f[i];
    }
    uint4 o;
    if constexpr (BF16) {
      o = pack_bf16x8(acc);
    } else {
      o.x = __float_as_uint(acc[0]);
      o.y = __float_as_uint(acc[1]);
      o.z = __float_as_uint(acc[2]);
      o.w = __float_as_uint(acc[3]);
    }
    __builtin_nontemporal_store(u32x4{o.x, o.y, o.z, o.w},
                                reinterpret_cast<u32x4*>(out + (size_t)t * row_chunks + c));
  }
}

}  // namespace

void launch_combine(const moe_config& c, const void* y_perm, const int32_t* a2r,
                    const float* w, const void* shared_y, void* out, hipStream_t s) {
  const bool bf16 = c.act_dtype == MOE_DT_BF16;
  const int row_chunks = c.H * (bf16 ? 2 : 4) / 16;
  const int64_t n = (int64_t)c.T * row_chunks;
  dim3 grid((unsigned)((n + 255) / 256));
  if (bf16)
    combine_kernel<true><<<grid, 256, 0, s>>>(
        reinterpret_cast<const uint4*>(y_perm), a2r, w,
        reinterpret_cast<const uint4*>(shared_y), c.T, c.k, row_chunks,
        reinterpret_cast<uint4*>(out));
  else
    combine_kernel<false><<<grid, 256, 0, s>>>(
        reinterpret_cast<const uint4*>(y_perm), a2r, w,
        reinterpret_cast<const uint4*>(shared_y), c.T, c.k, row_chunks,
        reinterpret_cast<uint4*>(out));
}

}  // namespace moe
