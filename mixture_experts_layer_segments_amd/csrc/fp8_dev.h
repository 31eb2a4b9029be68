// E4M3 encoding on the device, shared by the quantizers and the GEMM epilogue
// that writes E4M3 h (OCP 8-bit floating point, E4M3: bias 7, subnormals
// m * 2^-9, no infinity, max 448; one power-of-two scale per block, its
// exponent kept in the 8-bit E8M0 range of the FP8 matrix instructions).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace fp8_dev {

// E4M3 codes of four values, byte j = value j, each of magnitude at most
// 448 (a block scale makes it so): the hardware conversion, which rounds to
// the nearest E4M3 value, ties to even, keeps the sign of zeros and of values
// that round to zero, and on that range gives exactly the E4M3 definition.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Smallest s with amax <= 448 * 2^s (amax finite, >= 0); 0 for amax == 0;
// kept in [-127, 127], the range of the 8-bit power-of-two (E8M0) scales the
// FP8 matrix instructions take.  amax = (1 + m / 2^23) * 2^E and
// 448 = 1.75 * 2^8, so s = E - 8 when the mantissa is at most 0.75
// (m <= 0x600000), else E - 7.
__device__ __forceinline__ int block_exponent(float amax) {
  if (amax == 0.0f) return 0;
  int adj = 0;
  if (amax < 1.17549435e-38f) {              // fp32 subnormal: normalise exactly
    amax *= 18446744073709551616.0f;         // 2^64
    adj = -64;
  }
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)(b >> 23) - 127;
  const int s = E - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0) + adj;
  return max(-127, min(127, s));
}

// 2^s for s in [-127, 127], exactly (ldexpf of 1 would do; this states it).
__device__ __forceinline__ float pow2(int s) {
  return s >= -126 ? __uint_as_float((uint32_t)(s + 127) << 23) : __uint_as_float(0x00400000u);
}

}  // namespace fp8_dev
}  // namespace moe
