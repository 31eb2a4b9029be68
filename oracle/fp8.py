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

FP8 activations (the same page: tokens may be quantized to FP8 before
dispatch, and the low-precision expert GEMM): the plainest matching reading
is the same element format with one power-of-two scale per 1 x 128 block of
a row (each token's hidden vector in blocks of 128 along H; each expert's
hidden activation h in blocks of 128 along I).  h is the GEMM-1 result
rounded to bf16, as in the bf16 layer, before it is quantized: a quantized
code is an integer decided by a float, so it is decided on the value the
kernel holds.  Every scale exponent is kept in [-127, 127], the range of the
8-bit power-of-two (E8M0) scales that the FP8 matrix instructions take; a
block whose maximum is below 448 * 2^-127 keeps s = -127.

Everything is float64 on exact values: a power-of-two division and an E4M3
value are exact in float64, so the codes are a pure function of the inputs.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0      # largest finite E4M3 magnitude: 1.75 * 2^8
E4M3_NAN = 0x7F       # S.1111.111 (and 0xFF)
BLOCK = 128
S_MIN, S_MAX = -127, 127   # exponent range of an E8M0 scale


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


def scale_exponents(amax) -> np.ndarray:
    """block_exponents kept inside the E8M0 range [-127, 127]."""
    return np.clip(block_exponents(amax), S_MIN, S_MAX)


def quantize_blocks(w, block: int = BLOCK):
    """Codes uint8 [R, K] and power-of-two scales float64 [R/block, K/block]
    of one matrix w [R, K] (R and K multiples of ``block``)."""
    w = np.asarray(w, dtype=np.float64)
    R, K = w.shape
    assert R % block == 0 and K % block == 0, (R, K)
    blocks = w.reshape(R // block, block, K // block, block)
    s = scale_exponents(np.abs(blocks).max(axis=(1, 3)))            # [R/b, K/b]
    scaled = np.ldexp(blocks, -s[:, None, :, None])                 # exact
    codes = e4m3_encode(scaled).reshape(R, K)
    return codes, np.ldexp(1.0, s).astype(np.float64)


def dequantize_blocks(codes, scales, block: int = BLOCK) -> np.ndarray:
    """code * scale of every element (float64, exact)."""
    v = e4m3_decode(codes)
    return v * np.repeat(np.repeat(np.asarray(scales, np.float64), block, 0), block, 1)


# ------------------------------------------------------------ activations
def quantize_rows(x, block: int = BLOCK):
    """Codes uint8 [R, K] and power-of-two scales float64 [R, K/block] of
    activations x [R, K]: one scale per 1 x block piece of a row."""
    x = np.asarray(x, dtype=np.float64)
    R, K = x.shape
    assert K % block == 0, K
    pieces = x.reshape(R, K // block, block)
    s = scale_exponents(np.abs(pieces).max(axis=2))                 # [R, K/b]
    codes = e4m3_encode(np.ldexp(pieces, -s[:, :, None])).reshape(R, K)
    return codes, np.ldexp(1.0, s).astype(np.float64)


def dequantize_rows(codes, scales, block: int = BLOCK) -> np.ndarray:
    return e4m3_decode(codes) * np.repeat(np.asarray(scales, np.float64), block, 1)


def fake_quant_rows(x, block: int = BLOCK) -> np.ndarray:
    """The values the FP8 GEMMs multiply: dequantize(quantize_rows(x))."""
    return dequantize_rows(*quantize_rows(x, block), block)


def bf16_round(a) -> np.ndarray:
    """float64 -> the nearest bf16 value (via fp32, both steps to nearest
    even), as the GPU rounds its fp32 h."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def swiglu_hidden(x_rows, w13_e) -> np.ndarray:
    """silu(x W_gate) * (x W_up) of one expert (float64)."""
    I = w13_e.shape[0] // 2
    g = x_rows @ w13_e[:I].T
    u = x_rows @ w13_e[I:].T
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def expert_w8a8(xq_rows, w13_e, w2_e) -> np.ndarray:
    """One expert with FP8 activations: xq_rows are the quantized-dequantized
    input rows, w13_e / w2_e the dequantized FP8 weights; h is rounded to
    bf16 and quantized in 1 x 128 blocks before the down projection."""
    h = fake_quant_rows(bf16_round(swiglu_hidden(xq_rows, w13_e)))
    return h @ w2_e.T


def layer_forward_w8a8(cfg, logits, x64, w13_deq, w2_deq, sw13_deq=None, sw2_deq=None):
    """The layer with FP8 weights (already dequantized, float64) and FP8
    activations: x is quantized in 1 x 128 blocks before dispatch, each
    expert (and the shared one) runs expert_w8a8, and routing, permutation
    and combine are those of the bf16 layer."""
    from oracle import moe_oracle as orc
    ids, w, gap = orc.route(cfg, logits)
    p = orc.plan(cfg, ids)
    xq = fake_quant_rows(x64)
    r2t = p["row_to_token"]
    x_perm = np.where((r2t >= 0)[:, None], xq[np.maximum(r2t, 0)], 0.0)
    y = np.zeros((x_perm.shape[0], w2_deq.shape[1]))
    for s_, e in enumerate(p["seg_expert"].tolist()):
        r0, r1 = int(p["seg_offsets"][s_]), int(p["seg_offsets"][s_ + 1])
        if r1 > r0 and 0 <= e < w13_deq.shape[0]:
            y[r0:r1] = expert_w8a8(x_perm[r0:r1], w13_deq[e], w2_deq[e])
    shared_y = expert_w8a8(xq, sw13_deq, sw2_deq) if sw13_deq is not None else None
    out = orc.combine(y, p["assign_to_row"], w, shared_y)
    p.update(ids=ids, w=w, group_gap=gap, x_perm=x_perm, y_perm=y, shared_y=shared_y, out=out)
    return p


def token_outputs_w8a8(tokens, x64_rows, ids_rows, w_rows, expert_weights, shared=None):
    """Layer outputs of a few tokens straight from the definition with FP8
    activations (sampled checks at full size); ``expert_weights(e)`` returns
    the dequantized float64 (w13_e, w2_e)."""
    xq = fake_quant_rows(x64_rows)
    out = np.zeros((len(tokens), x64_rows.shape[1]))
    need = {}
    for i, _ in enumerate(tokens):
        for j, e in enumerate(ids_rows[i].tolist()):
            need.setdefault(e, []).append((i, j))
    for e, uses in sorted(need.items()):
        w13_e, w2_e = expert_weights(e)
        rows = np.array([i for i, _ in uses])
        y = expert_w8a8(xq[rows], w13_e, w2_e)
        for n, (i, j) in enumerate(uses):
            out[i] += w_rows[i, j] * y[n]
    if shared is not None:
        out += expert_w8a8(xq, shared[0], shared[1])
    return out
