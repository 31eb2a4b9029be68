// FP8 expert weights: block quantization to OCP E4M3 (the MoE inference
// blog, "Communication pressure": a low-precision GEMM kernel uses FP8 to cut
// memory and compute cost; element format from the OCP 8-bit floating point
// specification, E4M3: bias 7, subnormals m * 2^-9, no infinity, max 448).
//
// One workgroup per 128 x 128 block: the block maximum picks the power-of-two
// scale 2^s (the smallest s with max <= 448 * 2^s), then every element is
// rounded to the nearest E4M3 value of w / 2^s, ties to even (the hardware
// conversion; w / 2^s is exact in fp32 and at most 448 in magnitude), so the
// codes are a pure function of the input.
#include <math.h>

#include "fp8_dev.h"
#include "moe_internal.h"

namespace moe {
namespace {

using namespace fp8_dev;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Thread t of the block's 256 handles row t / 2, columns (t % 2) * 64 .. +64.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ src,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scale, int rows,
                                                           int cols) {
  __shared__ float wmax[4];
  const int bc = cols / 128, br = rows / 128;
  const int blk = blockIdx.x;
  const int mat = blk / (br * bc), rem = blk % (br * bc), bi = rem / bc, bj = rem % bc;
  const int t = threadIdx.x;
  const int row = bi * 128 + t / 2, col0 = bj * 128 + (t % 2) * 64;
  const size_t base = ((size_t)mat * rows + row) * cols + col0;

  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const u32x4*>(src + base + i * 8);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[i][j])), fabsf(bf16_hi(v[i][j]))));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int s = block_exponent(amax);
  if (t == 0) scale[((size_t)mat * br + bi) * bc + bj] = pow2(s);

  // 64 codes -> 16 words -> 4 x 16-byte stores (byte j of a word = column 4w + j)
  uint32_t out[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      out[i * 2 + j / 2] = e4m3x4(ldexpf(bf16_lo(v[i][j]), -s), ldexpf(bf16_hi(v[i][j]), -s),
                                  ldexpf(bf16_lo(v[i][j + 1]), -s),
                                  ldexpf(bf16_hi(v[i][j + 1]), -s));
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<u32x4*>(q + base + i * 16) =
        u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
}

// 8 E4M3 codes (byte j of word w = element 4w + j) times a power-of-two
// scale, as 8 bf16 (exact).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi, float sc) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true))};
}

// Activations: one power-of-two scale per 1 x 128 piece of a row.  A group
// of 16 lanes takes one piece (8 elements a lane, one 16-byte load), so a
// 256-thread block quantizes 16 pieces; the piece maximum is reduced over
// the group with lane shuffles.
// FAKE: instead of codes and scales, write each value to dst (which may be
// src: every element is read and written by the same lane) as its code
// times its scale, the bf16 value the codes stand for.
template <bool FAKE>
__global__ __launch_bounds__(256) void quantize_rows_fp8_kernel(const uint16_t* src,
                                                                uint8_t* __restrict__ q,
                                                                float* __restrict__ scale,
                                                                uint16_t* dst,
                                                                int64_t pieces, int cols) {
  const int64_t piece = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (piece >= pieces) return;                      // whole groups of 16 leave together
  const int sub = threadIdx.x & 15;
  const int pr = cols / 128;
  const int64_t row = piece / pr;
  const int col = (int)(piece % pr) * 128 + sub * 8;
  const size_t at = (size_t)row * cols + col;
  const u32x4 v = *reinterpret_cast<const u32x4*>(src + at);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(v[j])), fabsf(bf16_hi(v[j]))));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  const int s = block_exponent(amax);
  if (!FAKE && sub == 0) scale[piece] = pow2(s);
  uint32_t w[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    w[j] = e4m3x4(ldexpf(bf16_lo(v[2 * j]), -s), ldexpf(bf16_hi(v[2 * j]), -s),
                  ldexpf(bf16_lo(v[2 * j + 1]), -s), ldexpf(bf16_hi(v[2 * j + 1]), -s));
  }
  if constexpr (FAKE)
    *reinterpret_cast<u32x4*>(dst + at) = e4m3x8_to_bf16(w[0], w[1], pow2(s));
  else
    *reinterpret_cast<u32x2*>(q + at) = u32x2{w[0], w[1]};
}

// bf16 dst = codes times their 1 x 128 scales, 8 elements per thread.
__global__ __launch_bounds__(256) void dequantize_rows_fp8_kernel(const uint8_t* __restrict__ q,
                                                                  const float* __restrict__ scale,
                                                                  uint16_t* __restrict__ dst,
                                                                  int64_t pieces, int cols) {
  const int64_t piece = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (piece >= pieces) return;
  const int sub = threadIdx.x & 15;
  const int pr = cols / 128;
  const int64_t row = piece / pr;
  const int col = (int)(piece % pr) * 128 + sub * 8;
  const size_t at = (size_t)row * cols + col;
  const u32x2 c = *reinterpret_cast<const u32x2*>(q + at);
  *reinterpret_cast<u32x4*>(dst + at) = e4m3x8_to_bf16(c.x, c.y, scale[piece]);
}

}  // namespace

void launch_quantize_rows_fp8(int64_t rows, int cols, const void* src, uint8_t* q, float* scale,
                              hipStream_t s) {
  const int64_t pieces = rows * (cols / 128);
  if (pieces == 0) return;
  quantize_rows_fp8_kernel<false><<<(unsigned)((pieces + 15) / 16), 256, 0, s>>>(
      (const uint16_t*)src, q, scale, nullptr, pieces, cols);
}

void launch_dequantize_rows_fp8(int64_t rows, int cols, const uint8_t* q, const float* scale,
                                void* dst, hipStream_t s) {
  const int64_t pieces = rows * (cols / 128);
  if (pieces == 0) return;
  dequantize_rows_fp8_kernel<<<(unsigned)((pieces + 15) / 16), 256, 0, s>>>(
      q, scale, (uint16_t*)dst, pieces, cols);
}

void launch_fake_quant_rows_fp8(int64_t rows, int cols, void* data, hipStream_t s) {
  const int64_t pieces = rows * (cols / 128);
  if (pieces == 0) return;
  quantize_rows_fp8_kernel<true><<<(unsigned)((pieces + 15) / 16), 256, 0, s>>>(
      (const uint16_t*)data, nullptr, nullptr, (uint16_t*)data, pieces, cols);
}

void launch_quantize_fp8(int n_mat, int rows, int cols, const void* src, uint8_t* q,
                         float* scale, hipStream_t s) {
  const int64_t blocks = (int64_t)n_mat * (rows / 128) * (cols / 128);
  if (blocks == 0) return;
  quantize_fp8_kernel<<<(unsigned)blocks, 256, 0, s>>>((const uint16_t*)src, q, scale, rows,
                                                       cols);
}

}  // namespace moe
