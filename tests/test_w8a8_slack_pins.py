"""Pins of the W8A8 output check (tests/gpu_util.check_w8a8_out with
h_code_slack), on the CPU.

The GPU's W8A8 layer is compared with the oracle's within the bf16 tolerance
plus a per-element slack for h codes that sit on an fp32 rounding boundary.
A slack can hide mistakes, so here the check is fed whole-layer outputs that
are wrong in plausible ways, each built from the oracle's own pieces on the
small W8A8 layers the GPU tests run, and it must reject every one whose
output differs materially:

* h quantized without the bf16 rounding first,
* h not quantized at all,
* x not quantized before dispatch,
* h's piece scale one exponent too low (the piece maximum saturates),
* bf16 weights instead of their E4M3 values.

Two other mistakes -- pieces along the wrong axis (128 x 1 instead of
1 x 128) and a piece scale one exponent too high -- leave the output the
same to within a few 1e-6 of its maximum: with power-of-two scales the E4M3
grid is the same grid at every scale while the values stay in its normal
range, so only subnormal-range elements move.  No output tolerance can see
them, and this test states so (their distance is asserted to be tiny); the
bit-exact quantizer tests and the oracle's own FP8 pins (crafted pieces with
a subnormal tail) are what pin the axis and the exponent rule.
"""
import numpy as np
import pytest

from oracle import fp8 as ofp8
from tests import gpu_util as gu
from tests.test_gpu_w8a8 import SHAPES

# the small W8A8 layers whose whole oracle takes about a second each
CASES = ["w8a8_mid_split", "w8a8_big", "w8a8_grouped_shared", "w8a8_capacity_rings",
         "w8a8_decode_codes"]


def _layer_with(case, expert_fn, xq, w13=None, w2=None, sw13=None, sw2=None):
    """The oracle's layer with the oracle's routing and drops, but each
    expert computed by expert_fn(x rows, w13_e, w2_e)."""
    c, r = case.cfg, case.ref
    w13 = case.w13_64 if w13 is None else w13
    w2 = case.w2_64 if w2 is None else w2
    out = np.zeros((c.T, c.H))
    kept = r["assign_to_row"].reshape(c.T, c.k) >= 0
    for e in range(c.E):
        t, j = np.nonzero((r["ids"] == e) & kept)
        if t.size:
            out[t] += r["w"][t, j][:, None] * expert_fn(xq[t], w13[e], w2[e])
    if c.shared_I:
        out += expert_fn(xq, case.sw13_64 if sw13 is None else sw13,
                         case.sw2_64 if sw2 is None else sw2)
    return out


def _h(xq, w13):
    return ofp8.swiglu_hidden(xq, w13)


def _rows_scaled(h, shift):
    """h quantized in 1 x 128 pieces with every scale exponent moved by shift."""
    _, sc = ofp8.quantize_rows(h)
    s = (np.log2(sc) + shift).astype(np.int64)
    n = h.shape[0]
    codes = ofp8.e4m3_encode(np.ldexp(h.reshape(n, -1, 128), -s[:, :, None]))
    return ofp8.e4m3_decode(codes.reshape(h.shape)) * np.repeat(2.0 ** s, 128, axis=1)


def _cols(h):
    """h quantized in 128 x 1 pieces (down the rows) instead of 1 x 128."""
    n = h.shape[0]
    hp = np.vstack([h, np.zeros(((-n) % 128, h.shape[1]))])
    return ofp8.fake_quant_rows(hp.T).T[:n]


WRONG = {
    "h not rounded to bf16": lambda xq, a, b: ofp8.fake_quant_rows(_h(xq, a)) @ b.T,
    "h not quantized": lambda xq, a, b: ofp8.bf16_round(_h(xq, a)) @ b.T,
    "h scale one exponent low": lambda xq, a, b: _rows_scaled(ofp8.bf16_round(_h(xq, a)), -1) @ b.T,
}
INVISIBLE = {
    "h in 128 x 1 pieces": lambda xq, a, b: _cols(ofp8.bf16_round(_h(xq, a))) @ b.T,
    "h scale one exponent high": lambda xq, a, b: _rows_scaled(ofp8.bf16_round(_h(xq, a)), 1) @ b.T,
}


@pytest.fixture(scope="module", params=CASES)
def case(request):
    c = gu.SmallCase(SHAPES[request.param])
    return c, gu.w8a8_slack(c), ofp8.fake_quant_rows(c.x64)


def test_the_oracle_layer_itself_passes(case):
    c, slack, xq = case
    got = _layer_with(c, ofp8.expert_w8a8, xq)
    gu.check_w8a8_out(got, c.ref["out"], slack, c.cfg.name + " oracle vs itself")


@pytest.mark.parametrize("mistake", sorted(WRONG))
def test_wrong_h_handling_is_rejected(case, mistake):
    c, slack, xq = case
    got = _layer_with(c, WRONG[mistake], xq)
    with pytest.raises(AssertionError):
        gu.check_w8a8_out(got, c.ref["out"], slack, f"{c.cfg.name}: {mistake}")


def test_unquantized_x_is_rejected(case):
    c, slack, _ = case
    got = _layer_with(c, ofp8.expert_w8a8, c.x64)
    with pytest.raises(AssertionError):
        gu.check_w8a8_out(got, c.ref["out"], slack, c.cfg.name + ": x not quantized")


def test_bf16_weights_instead_of_e4m3_are_rejected(case):
    c, slack, xq = case
    import moe_inputs as mi
    cfg = c.cfg
    w13 = np.stack([mi.values_f64(mi.w13(cfg, e), "bf16") for e in range(cfg.E)])
    w2 = np.stack([mi.values_f64(mi.w2(cfg, e), "bf16") for e in range(cfg.E)])
    sw13 = mi.values_f64(mi.shared_w13(cfg), "bf16") if cfg.shared_I else None
    sw2 = mi.values_f64(mi.shared_w2(cfg), "bf16") if cfg.shared_I else None
    got = _layer_with(c, ofp8.expert_w8a8, xq, w13, w2, sw13, sw2)
    with pytest.raises(AssertionError):
        gu.check_w8a8_out(got, c.ref["out"], slack, cfg.name + ": bf16 weights")


@pytest.mark.parametrize("mistake", sorted(INVISIBLE))
def test_scale_invariant_mistakes_do_not_move_the_output(case, mistake):
    c, _, xq = case
    got = _layer_with(c, INVISIBLE[mistake], xq)
    ref = c.ref["out"]
    assert np.abs(got - ref).max() <= 1e-4 * np.abs(ref).max()


def test_slack_stays_a_small_fraction(case):
    """The slack exceeds the plain tolerance on at most 1% of the elements."""
    c, slack, _ = case
    m = np.abs(c.ref["out"]).max()
    assert np.mean(slack > gu.BF16_REL * m) <= gu.W8A8_BIG_SLACK_FRAC
