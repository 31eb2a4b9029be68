"""CPU oracle for FP8 expert weights -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP product path never calls it and
shares no code with it.

The pages name low-precision expert GEMMs ("Mixture-of-Experts Inference:
parallelism, communication, and load balancing", section "Communication
pressure", its list of optimized kernels for MoE: a low-precision GEMM kernel
uses FP8 or FP4 to cut compute and memory cost) but fix no format.  The
reading taken here, the plainest that keeps the layer's arithmetic otherwise
unchanged:

* element format: OCP 8-bit floating point E4M3 (the "OFP8" specification):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
  holds subnormals m * 2^-9; S.1111.111 is NaN; there is no infinity; the
  largest finite magnitude is 448;
* scaling: every expert matrix (W13[e] rows x H, W2[e] rows x I) is cut into
  128 x 128 blocks, each with one power-of-two scale 2^s, s the smallest
  integer with max|block| <= 448 * 2^s (s = 0 for an all-zero block);
* elements: code = E4M3 round-to-nearest-even of w / 2^s (exact division);
* the layer then runs on the dequantized weights code * 2^s with bf16
  activations, exactly as with bf16 weights.

Everything is float64 on exact values: a power-of-two division and an E4M3
value are exact in float64, so the codes are a pure function of the inputs.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0      # largest finite E4M3 magnitude: 1.75 * 2^8
E4M3_NAN = 0x7F       # S.1111.111 (and 0xFF)
BLOCK = 128


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (float64; NaN codes give NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(y) -> np.ndarray:
    """Round-to-nearest-even E4M3 code of each value (the sign bit follows the
    input's, so -0.0 gives 0x80); magnitudes beyond 448 saturate to 448 (the
    block scaling below never produces them)."""
    y = np.asarray(y, dtype=np.float64)
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    # normal range: a = f * 2^E with f in [0.5, 1), so floor(log2 a) = E - 1
    _, E = np.frexp(a)
    ex = E.astype(np.int64) - 1
    n = np.rint(np.ldexp(a, 3 - ex)).astype(np.int64)      # in [8, 16], ties to even
    carry = n == 16
    ex = np.where(carry, ex + 1, ex)
    n = np.where(carry, 8, n)
    sat = (ex > 8) | ((ex == 8) & (n > 14))
    ex = np.where(sat, 8, ex)
    n = np.where(sat, 14, n)
    normal = sign | ((ex + 7) << 3) | (n - 8)
    # subnormal range (a < 2^-6): quantum 2^-9; 8 quanta is the smallest normal
    ns = np.rint(np.ldexp(a, 9)).astype(np.int64)             # in [0, 8], ties to even
    sub = sign | ns
    return np.where(a < 2.0 ** -6, sub, normal).astype(np.uint8)


def block_exponent(amax: float) -> int:
    """Smallest integer s with amax <= 448 * 2^s; 0 when amax == 0."""
    if amax == 0.0:
        return 0
    s = math.ceil(math.log2(amax / E4M3_MAX))
    # the logarithm may round: settle s on the definition itself
    while amax > E4M3_MAX * 2.0 ** s:
        s += 1
    while amax <= E4M3_MAX * 2.0 ** (s - 1):
        s -= 1
    return s


def block_exponents(amax) -> np.ndarray:
    """block_exponent of every element of amax (vectorised): with
    amax = f * 2^E, f in [0.5, 1), 448 * 2^s >= amax first holds at
    s = E - 9 when f <= 0.875 (448 = 0.875 * 2^9), else at s = E - 8."""
    a = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(a)
    s = E.astype(np.int64) - 9 + (f > 0.875)
    return np.where(a == 0.0, 0, s)


def quantize_blocks(w, block: int = BLOCK):
    """Codes uint8 [R, K] and power-of-two scales float64 [R/block, K/block]
    of one matrix w [R, K] (R and K multiples of ``block``)."""
    w = np.asarray(w, dtype=np.float64)
    R, K = w.shape
    assert R % block == 0 and K % block == 0, (R, K)
    blocks = w.reshape(R // block, block, K // block, block)
    s = block_exponents(np.abs(blocks).max(axis=(1, 3)))            # [R/b, K/b]
    scaled = np.ldexp(blocks, -s[:, None, :, None])                 # exact
    codes = e4m3_encode(scaled).reshape(R, K)
    return codes, np.ldexp(1.0, s).astype(np.float64)


def dequantize_blocks(codes, scales, block: int = BLOCK) -> np.ndarray:
    """code * scale of every element (float64, exact)."""
    v = e4m3_decode(codes)
    return v * np.repeat(np.repeat(np.asarray(scales, np.float64), block, 0), block, 1)
