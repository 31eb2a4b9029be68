"""Pins of the FP8 weight oracle (CPU only).

Every pin rests on something other than the oracle itself: the encodings
the OCP 8-bit floating point specification (OFP8) tabulates for E4M3,
brute force over the 254 finite codes, the definition of the block scale
checked by linear search, and exact reconstruction of matrices built from
E4M3 values.  The last test plants plausible mistakes in the oracle and
checks that some pin fails for each.
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


# ------------------------------------------------------------ planted mistakes
PINS = [test_finite_codes_are_distinct_monotone_and_round_trip, test_midpoints_round_to_even_codes,
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


@pytest.mark.parametrize("name,fn", [("e4m3_encode", _ties_away), ("e4m3_decode", _bias8_decode),
                                     ("block_exponent", _floor_exponent),
                                     ("e4m3_encode", _truncate),
                                     ("block_exponents", _exponents_off_by_one)],
                         ids=["ties_away", "bias8_decode", "floor_exponent", "truncate",
                              "exponents_off_by_one"])
def test_planted_mistake_is_caught(name, fn):
    failed = 0
    with _planted(name, fn):
        for pin in PINS:
            try:
                pin()
            except Exception:
                failed += 1
    assert failed, f"no pin catches {fn.__name__}"
