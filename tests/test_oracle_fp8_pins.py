"""Pins of the FP8 oracle, weights and activations (CPU only).

Every pin rests on something other than the oracle itself: the encodings
the OCP 8-bit floating point specification (OFP8) tabulates for E4M3,
brute force over the 254 finite codes, the definition of the block scale
checked by linear search, exact reconstruction of matrices built from
E4M3 values, torch's bf16 rounding, a hand-worked one-expert layer and a
layer whose every value sits on the E4M3 grid (where the FP8 layer must
equal the plain one).  The last test plants plausible mistakes in the oracle
and checks that some pin fails for each.
"""
import contextlib
import math

import numpy as np
import pytest

from oracle import fp8

POS = np.arange(0x00, 0x7F, dtype=np.uint8)          # +0 .. 448 (0x7F is NaN)


def _table():
    v = fp8.e4m3_decode(POS)
    return POS, v


# ------------------------------------------------------------ OFP8 facts
@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x80, -0.0),
    (0x01, 2.0 ** -9),                 # smallest subnormal
    (0x07, 0.875 * 2.0 ** -6),         # largest subnormal
    (0x08, 2.0 ** -6),                 # smallest normal
    (0x38, 1.0), (0x40, 2.0), (0x30, 0.5),
    (0x7E, 448.0), (0xFE, -448.0),     # largest finite
    (0x77, 240.0), (0x3F, 1.875),
])
def test_ofp8_table_values(code, value):
    got = fp8.e4m3_decode([code])[0]
    assert got == value and math.copysign(1, got) == math.copysign(1, value)
    assert fp8.e4m3_encode([value])[0] == code


def test_nan_codes_and_no_infinity():
    v = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(np.delete(v, [0x7F, 0xFF])).all()


def test_finite_codes_are_distinct_monotone_and_round_trip():
    codes, v = _table()
    assert np.all(np.diff(v) > 0)                     # monotone in the code
    assert np.array_equal(fp8.e4m3_encode(v), codes)
    neg = fp8.e4m3_decode(codes | 0x80)
    assert np.array_equal(neg, -v)
    assert np.array_equal(fp8.e4m3_encode(neg[1:]), (codes | 0x80)[1:])


def test_midpoints_round_to_even_codes():
    """Halfway between two neighbouring values the even code wins (the even
    code is the one whose mantissa ends in 0)."""
    codes, v = _table()
    mid = (v[:-1] + v[1:]) / 2
    got = fp8.e4m3_encode(mid)
    want = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(got, want)


def test_nearest_value_by_brute_force():
    codes, v = _table()
    rng = np.random.default_rng(7)
    y = np.concatenate([rng.uniform(0, 448, 4000), rng.uniform(0, 2 ** -5, 2000),
                        rng.uniform(0, 1, 2000)])
    got = fp8.e4m3_decode(fp8.e4m3_encode(y))
    err = np.abs(y[:, None] - v[None, :])
    best = v[np.argmin(err, axis=1)]
    # where two values are equally near, either is nearest; the midpoint pin fixes which
    assert np.all(np.abs(y - got) == np.min(err, axis=1))
    assert np.mean(got == best) > 0.999


def test_saturation():
    assert fp8.e4m3_encode([500.0, 1e9, -1e9])[0] == 0x7E
    assert fp8.e4m3_encode([1e9])[0] == 0x7E and fp8.e4m3_encode([-1e9])[0] == 0xFE


# ------------------------------------------------------------ block scale
def _brute_exponent(amax):
    for s in range(-160, 160):
        if amax <= 448.0 * 2.0 ** s:
            return s
    raise AssertionError


def test_block_exponent_definition():
    assert fp8.block_exponent(448.0) == 0
    assert fp8.block_exponent(449.0) == 1
    assert fp8.block_exponent(1.0) == -8          # 256 <= 448 < 512
    assert fp8.block_exponent(448.0 * 2 ** -5) == -5
    assert fp8.block_exponent(0.0) == 0
    rng = np.random.default_rng(3)
    for a in np.concatenate([np.exp(rng.uniform(-40, 40, 300)), 448.0 * 2.0 ** np.arange(-30, 30)]):
        assert fp8.block_exponent(float(a)) == _brute_exponent(float(a)), a


def test_vectorised_exponents_follow_the_definition():
    rng = np.random.default_rng(4)
    a = np.concatenate([np.exp(rng.uniform(-60, 60, 2000)), 448.0 * 2.0 ** np.arange(-40, 40),
                        np.nextafter(448.0 * 2.0 ** np.arange(-40, 40), np.inf),
                        np.nextafter(448.0 * 2.0 ** np.arange(-40, 40), 0), [0.0]])
    got = fp8.block_exponents(a)
    assert all(int(g) == (0 if x == 0 else _brute_exponent(float(x))) for g, x in zip(got, a))


def test_block_quantization_uses_the_range_and_bounds_the_error():
    rng = np.random.default_rng(11)
    w = rng.normal(0, 0.02, size=(256, 384))
    w[128:, 128:256] *= 1e3                          # one block on another scale
    codes, scales = fp8.quantize_blocks(w)
    assert scales.shape == (2, 3)
    assert np.all(np.log2(scales) == np.round(np.log2(scales)))
    deq = fp8.dequantize_blocks(codes, scales)
    for bi in range(2):
        for bj in range(3):
            blk = np.s_[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            top = np.max(np.abs(w[blk])) / scales[bi, bj]
            assert 224.0 < top <= 448.0               # the scale is the smallest that fits
            a = np.abs(w[blk])
            normal = a >= 2.0 ** -6 * scales[bi, bj]
            # half an ulp of a 3-bit mantissa: relative 2^-4; absolute 2^-10 * scale below
            assert np.all(np.abs(deq[blk] - w[blk])[normal] <= 2.0 ** -4 * a[normal])
            assert np.all(np.abs(deq[blk] - w[blk])[~normal] <= 2.0 ** -10 * scales[bi, bj])


def test_exact_reconstruction_of_e4m3_matrices():
    codes, v = _table()
    rng = np.random.default_rng(5)
    base = rng.choice(np.concatenate([v, -v[1:]]), size=(128, 256))
    base[0, 0] = 448.0                               # each block reaches the top code
    base[0, 128] = -448.0
    w = base * 2.0 ** np.array([[-7.0, 3.0]]).repeat(128, 0).repeat(128, 1)
    c, s = fp8.quantize_blocks(w)
    assert np.array_equal(s, np.array([[2.0 ** -7, 2.0 ** 3]]))
    assert np.array_equal(fp8.dequantize_blocks(c, s), w)


def test_zero_block():
    c, s = fp8.quantize_blocks(np.zeros((128, 128)))
    assert s[0, 0] == 1.0 and not c.any()


# ------------------------------------------------------------ activations
def test_row_blocks_are_weight_blocks_of_one_row():
    """A 1 x 128 piece of a row is quantized exactly as a 128 x 128 weight
    block whose other rows are zero (the zeros do not change the maximum)."""
    rng = np.random.default_rng(12)
    x = rng.normal(0, 1.0, size=(5, 384)) * 2.0 ** rng.integers(-20, 20, size=(5, 1))
    x[2, 128:256] = 0.0
    codes, scales = fp8.quantize_rows(x)
    assert codes.shape == (5, 384) and scales.shape == (5, 3)
    for r in range(5):
        pad = np.zeros((128, 384))
        pad[0] = x[r]
        c_ref, s_ref = fp8.quantize_blocks(pad)
        assert np.array_equal(codes[r], c_ref[0]) and np.array_equal(scales[r], s_ref[0])
    assert np.array_equal(fp8.dequantize_rows(codes, scales),
                          fp8.e4m3_decode(codes) * np.repeat(scales, 128, 1))


def test_scale_exponents_stay_in_the_e8m0_range():
    """amax = 448 * 2^-128 would want s = -128; the E8M0 scale stops at
    -127, so the block keeps 2^-127 and values below half its smallest
    subnormal step (2^-137) become zero."""
    assert fp8.block_exponent(448.0 * 2.0 ** -128) == -128
    assert fp8.scale_exponents(np.array([448.0 * 2.0 ** -128, 448.0 * 2.0 ** -127, 1.0])).tolist() \
        == [-127, -127, -8]
    x = np.zeros((1, 128))
    x[0, :3] = [2.0 ** -130, 2.0 ** -138, -2.0 ** -129]
    codes, scales = fp8.quantize_rows(x)
    assert scales[0, 0] == 2.0 ** -127
    assert fp8.dequantize_rows(codes, scales)[0, :3].tolist() == [2.0 ** -130, 0.0, -2.0 ** -129]
    w = np.zeros((128, 128))
    w[0, 0] = 2.0 ** -131
    c, sc = fp8.quantize_blocks(w)
    assert sc[0, 0] == 2.0 ** -127 and fp8.dequantize_blocks(c, sc)[0, 0] == 2.0 ** -131


def test_bf16_round_matches_torch():
    import torch
    rng = np.random.default_rng(13)
    a = np.concatenate([rng.normal(0, 1, 5000) * 2.0 ** rng.integers(-30, 30, 5000),
                        (1 + np.arange(256) / 256.0 + 2.0 ** -9), [0.0, -0.0, 1.0]])
    want = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(fp8.bf16_round(a), want)


def _one_expert_case():
    """T = 1, E = k = 1, H = I = 128: x = 1.1875 e_0; W_gate[:, 0] = 80,
    W_up[:, 0] = 1.75 * 2^-6, other weights of W13 zero; W2 from E4M3 values.
    Quantized x: 1.1875 * 256 = 304 lies halfway between the E4M3 values 288
    and 320, and the even one is 320, so x -> 1.25; g = 1.25 * 80 = 100
    (silu(100) = 100 in float64) and u = 1.25 * 1.75 * 2^-6, so
    h = 3.41796875 for every i, 3.421875 in bf16; the row's scale is 2^-7
    (3.421875 <= 448 * 2^-7 = 3.5), 3.421875 * 128 = 438 and the nearest
    E4M3 value is 448, so h -> 3.5.  out = 3.5 * sum_i W2[:, i].  (Unquantized
    x would give h -> 3.0, an unquantized h 3.421875.)"""
    import moe_inputs as mi
    cfg = mi.MoEShape("w8a8", T=1, H=128, E=1, k=1, I=128, weights="fp8")
    x = np.zeros((1, 128))
    x[0, 0] = 1.1875
    w13 = np.zeros((1, 256, 128))
    w13[0, :128, 0] = 80.0
    w13[0, 128:, 0] = 1.75 * 2.0 ** -6
    codes = np.array([0x38, 0x40, 0xB8, 0x30, 0x44, 0xC2])          # 1, 2, -1, 0.5, 2.5, -2.25
    rng = np.random.default_rng(14)
    w2 = fp8.e4m3_decode(rng.choice(codes, size=(1, 128, 128))) * 2.0 ** -4
    w2[0, 0, 0] = 2.5 * 2.0 ** -4                                    # keeps the block scale 2^-9
    return cfg, x, w13, w2


def test_w8a8_layer_hand_example():
    cfg, x, w13, w2 = _one_expert_case()
    w13d = fp8.dequantize_blocks(*fp8.quantize_blocks(w13[0]))[None]
    w2d = fp8.dequantize_blocks(*fp8.quantize_blocks(w2[0]))[None]
    assert np.array_equal(w13d, w13) and np.array_equal(w2d, w2)      # exact weights
    r = fp8.layer_forward_w8a8(cfg, np.zeros((1, 1), np.float32), x, w13d, w2d)
    assert r["w"][0, 0] == 1.0
    np.testing.assert_allclose(r["out"][0], 3.5 * w2[0].sum(axis=1), rtol=1e-15, atol=0)
    # with a shared expert of the same weights, its output adds once more
    r2 = fp8.layer_forward_w8a8(cfg, np.zeros((1, 1), np.float32), x, w13d, w2d, w13d[0], w2d[0])
    np.testing.assert_allclose(r2["out"][0], 7.0 * w2[0].sum(axis=1), rtol=1e-15, atol=0)


def test_w8a8_layer_equals_the_bf16_layer_when_every_value_is_on_the_grid():
    """One-hot rows times powers of two, gate weights in [48, 96] (silu is the
    identity there in float64), up weights powers of two: x, the weights and
    h all sit on the E4M3 grid of their blocks, so every quantization is
    exact and the FP8 layer must equal the plain layer on the same values."""
    import moe_inputs as mi
    from oracle import moe_oracle as orc
    T, H, E, k, I = 24, 128, 4, 2, 128
    cfg = mi.MoEShape("grid", T=T, H=H, E=E, k=k, I=I, weights="fp8", shared_I=128)
    rng = np.random.default_rng(15)
    x = np.zeros((T, H))
    x[np.arange(T), rng.integers(0, H, T)] = rng.choice([1.0, 2.0], T)
    gate = rng.choice([48.0, 56.0, 64.0, 80.0, 96.0], size=(E + 1, I, H))
    up = rng.choice([1.0, -1.0, 0.5, -0.5], size=(E + 1, I, H)) * 2.0 ** -4
    w13 = np.concatenate([gate, up], axis=1)
    w2 = rng.choice([1.0, -1.25, 1.5, -1.75], size=(E + 1, H, I)) * 2.0 ** -6
    for m in list(w13) + list(w2):
        assert np.array_equal(fp8.dequantize_blocks(*fp8.quantize_blocks(m)), m)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    a = fp8.layer_forward_w8a8(cfg, lg, x, w13[:E], w2[:E], w13[E], w2[E])
    b = orc.layer_forward(cfg, lg, x, w13[:E], w2[:E], w13[E], w2[E])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-13, atol=1e-13)
    assert np.abs(b["out"]).max() > 1.0


# ------------------------------------------------------------ planted mistakes
PINS = [test_row_blocks_are_weight_blocks_of_one_row, test_scale_exponents_stay_in_the_e8m0_range,
        test_bf16_round_matches_torch, test_w8a8_layer_hand_example,
        test_w8a8_layer_equals_the_bf16_layer_when_every_value_is_on_the_grid,
        test_finite_codes_are_distinct_monotone_and_round_trip, test_midpoints_round_to_even_codes,
        test_nearest_value_by_brute_force, test_saturation, test_block_exponent_definition,
        test_vectorised_exponents_follow_the_definition,
        test_block_quantization_uses_the_range_and_bounds_the_error,
        test_exact_reconstruction_of_e4m3_matrices, test_zero_block,
        lambda: [test_ofp8_table_values(c, v) for c, v in
                 [(0x01, 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x7E, 448.0), (0x77, 240.0)]]]

_orig_encode, _orig_decode, _orig_exp = fp8.e4m3_encode, fp8.e4m3_decode, fp8.block_exponent
_orig_exps = fp8.block_exponents


def _ties_away(y):
    y = np.asarray(y, dtype=np.float64)
    codes, v = _table()
    a = np.minimum(np.abs(y), 448.0)
    idx = np.searchsorted(v, a)                      # first value >= a
    idx = np.clip(idx, 0, len(v) - 1)
    lo = np.clip(idx - 1, 0, len(v) - 1)
    pick = np.where(np.abs(v[idx] - a) <= np.abs(a - v[lo]), idx, lo)
    return (codes[pick] | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def _bias8_decode(codes):
    return _orig_decode(codes) / 2.0


def _floor_exponent(amax):
    return 0 if amax == 0 else math.floor(math.log2(amax / 448.0))


def _exponents_off_by_one(amax):
    return _orig_exps(amax) - 1


def _truncate(y):
    y = np.asarray(y, dtype=np.float64)
    codes, v = _table()
    a = np.minimum(np.abs(y), 448.0)
    idx = np.clip(np.searchsorted(v, a, side="right") - 1, 0, len(v) - 1)
    return (codes[idx] | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


@contextlib.contextmanager
def _planted(name, fn):
    orig = getattr(fp8, name)
    setattr(fp8, name, fn)
    try:
        yield
    finally:
        setattr(fp8, name, orig)


_orig_expert, _orig_qrows = fp8.expert_w8a8, fp8.quantize_rows


def _h_not_quantized(xq_rows, w13_e, w2_e):
    return fp8.bf16_round(fp8.swiglu_hidden(xq_rows, w13_e)) @ w2_e.T


def _columns_as_blocks(x, block=128):
    codes, scales = _orig_qrows(np.asarray(x).T, block)   # 128 x 1 pieces: wrong axis
    return codes.T, np.repeat(scales.T, 1, 0)


def _no_clamp(amax):
    return fp8.block_exponents(amax)


def _no_activation_quantization(x, block=128):
    return np.asarray(x, dtype=np.float64)


@pytest.mark.parametrize("name,fn", [("e4m3_encode", _ties_away), ("e4m3_decode", _bias8_decode),
                                     ("block_exponent", _floor_exponent),
                                     ("e4m3_encode", _truncate),
                                     ("block_exponents", _exponents_off_by_one),
                                     ("expert_w8a8", _h_not_quantized),
                                     ("quantize_rows", _columns_as_blocks),
                                     ("scale_exponents", _no_clamp),
                                     ("fake_quant_rows", _no_activation_quantization)],
                         ids=["ties_away", "bias8_decode", "floor_exponent", "truncate",
                              "exponents_off_by_one", "h_not_quantized", "columns_as_blocks",
                              "no_clamp", "no_activation_quantization"])
def test_planted_mistake_is_caught(name, fn):
    failed = 0
    with _planted(name, fn):
        for pin in PINS:
            try:
                pin()
            except Exception:
                failed += 1
    assert failed, f"no pin catches {fn.__name__}"
