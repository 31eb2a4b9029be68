"""GPU parity of the FP8-activation (W8A8) path against the oracle.

* moe_quantize_act_fp8: codes and 1 x 128 scales bit for bit against the
  oracle's quantize_rows -- random rows over many scales (zero pieces,
  subnormal-range elements, negative zeros), every finite bf16 value in
  [-448, 448], and pieces small enough that the scale exponent stops at -127;
  the weight quantizer's clamp at -127 likewise.
* moe_layer_forward_w8a8 / moe_grouped_ffn_w8a8 on small layers spanning the
  weight-streaming decode tiles (activations dequantized on load) and the
  FP8 x FP8 ring tiles (mid and big shapes, splits, groups, a shared expert,
  the capacity layout): routing bit for bit, outputs within the bf16 layer
  tolerance of the oracle's W8A8 layer on its own quantization of the same
  drawn weights, plus a slack for h codes that may legitimately differ: the
  oracle decides h's codes on bf16 values it rounds from float64 sums, the
  GPU on bf16 values rounded from fp32 sums, so where an element sits within
  the fp32 rounding band of a code boundary either code is correct (as
  either group is correct at a routing tie).  The slack is one E4M3 step of
  exactly those elements, times |W2| (tests/gpu_util.h_code_slack); every
  other element must match within the plain tolerance.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import fp8 as ofp8
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_segments_amd as m
    return m


def _act_codes(moe, bits):
    """bits: bf16 bit patterns [R, C] -> compare the library's activation
    codes and scales with the oracle's, exactly."""
    src = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(gu.dev()).view(torch.bfloat16)
    q, sc = gu.quantize_act(moe, src)
    torch.cuda.synchronize()
    c_ref, s_ref = ofp8.quantize_rows(mi.values_f64(bits, "bf16"))
    c_got = q.cpu().numpy()
    bad = np.argwhere(c_got != c_ref)
    assert bad.size == 0, (bad[:5], c_got[tuple(bad[0])], c_ref[tuple(bad[0])])
    assert np.array_equal(sc.cpu().numpy().astype(np.float64), s_ref)


def test_act_quantizer_random_scales(moe):
    rng = np.random.default_rng(31)
    x = rng.normal(0, 1.0, size=(37, 640))
    x *= np.repeat(2.0 ** rng.integers(-40, 40, size=(37, 5)), 128, axis=1)
    x[3, :128] = 0.0                                           # all-zero piece
    x[5, 128:256] *= np.where(rng.random(128) < 0.5, 2.0 ** -12, 1.0)
    x[7, 9] = -0.0
    x[8, 256:384] = np.round(x[8, 256:384] * 4) / 4
    _act_codes(moe, mi.bf16_bits(x.astype(np.float32)))


def test_act_quantizer_every_bf16_in_range(moe):
    pos = np.arange(0, 0x43E1, dtype=np.uint32)
    allv = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    n = -(-allv.size // 127)
    flat = np.zeros((n, 128), dtype=np.uint16)
    for b in range(n):
        chunk = allv[b * 127:(b + 1) * 127]
        flat[b, 0] = 0x43E0                                    # 448: scale 1 in every piece
        flat[b, 1:1 + chunk.size] = chunk
    _act_codes(moe, flat)


def test_scale_exponent_clamp(moe):
    """Pieces and blocks whose maximum is below 448 * 2^-127 keep scale 2^-127
    (the bf16 values here are fp32 subnormals, down to 2^-133)."""
    x = np.zeros((2, 256), dtype=np.float64)
    x[0, :4] = [2.0 ** -130, 2.0 ** -133, -2.0 ** -129, 3 * 2.0 ** -131]
    x[1, 128:130] = [2.0 ** -127, 2.0 ** -126]
    bits = mi.bf16_bits(x.astype(np.float32))
    _act_codes(moe, bits)
    w = np.zeros((1, 128, 128))
    w[0, 0, :3] = [2.0 ** -131, 2.0 ** -132, 2.0 ** -129]
    wb = mi.bf16_bits(w.astype(np.float32))
    src = torch.from_numpy(wb.view(np.int16)).to(gu.dev()).view(torch.bfloat16)
    q, sc = gu.quantize_fp8(moe, src)
    torch.cuda.synchronize()
    c_ref, s_ref = ofp8.quantize_blocks(mi.values_f64(wb[0], "bf16"))
    assert s_ref[0, 0] == 2.0 ** -127
    assert np.array_equal(q[0].cpu().numpy(), c_ref)
    assert sc[0].cpu().numpy()[0, 0] == np.float32(2.0 ** -127)


SHAPES = {
    # weight-streaming decode tiles: activations dequantized on load
    "w8a8_decode": mi.MoEShape("a1", T=40, H=1024, E=32, k=2, I=512, weights="fp8", acts="fp8",
                               seed=51),
    "w8a8_decode_shared_grouped": mi.MoEShape("a2", T=24, H=2048, E=16, k=2, I=512,
                                              score="sigmoid", n_group=4, topk_group=2,
                                              shared_I=1024, weights="fp8", acts="fp8", seed=52),
    # the grouped FFN alone takes the decode tiles (120 rows over 8 segments)
    # but the workspace, sized for the layer with its shared expert (180 rows
    # over 9 segments: ring tiles), holds no bf16 copy of the activations, so
    # the E4M3-activation decode tiles run
    "w8a8_decode_codes": mi.MoEShape("a7", T=60, H=512, E=8, k=2, I=512, shared_I=512,
                                     weights="fp8", acts="fp8", seed=57),
    # FP8 x FP8 ring tiles: 128 x 256 with replica splits and N / K tails
    "w8a8_mid_split": mi.MoEShape("a3", T=300, H=640, E=16, k=4, I=384, zipf_s=1.2,
                                  n_hot_split=3, split_ways=2, weights="fp8", acts="fp8",
                                  seed=53),
    # 256 x 256 ring tiles
    "w8a8_big": mi.MoEShape("a4", T=1100, H=384, E=3, k=1, I=256, zipf_s=1.0, weights="fp8",
                            acts="fp8", seed=54),
    # groups, a shared expert, ring tiles
    "w8a8_grouped_shared": mi.MoEShape("a5", T=200, H=256, E=32, k=4, I=128, score="sigmoid",
                                       n_group=4, topk_group=2, shared_I=256, zipf_s=1.0,
                                       weights="fp8", acts="fp8", seed=55),
    # the fixed-capacity layout
    "w8a8_capacity_rings": mi.MoEShape("a6", T=300, H=512, E=16, k=4, I=256, zipf_s=1.2,
                                       capacity_factor_permille=1000, weights="fp8", acts="fp8",
                                       seed=56),
}


@pytest.fixture(scope="module", params=sorted(SHAPES))
def case(request):
    print(f"\n[w8a8 case] {request.param}", flush=True)
    return gu.SmallCase(SHAPES[request.param])


def test_layer_forward_w8a8(moe, case):
    c = case.cfg
    o = gu.run_layer(moe, c, case.device_inputs())
    for name, (codes, scales) in case.q.items():
        got = o["q"][name]
        got = got if got.dim() == 3 else got[None]
        assert np.array_equal(got.cpu().numpy(), codes), name
    r = case.ref
    mism = gu.check_routing(c, o["ids"].cpu().numpy(), o["w"].cpu().numpy(), r["ids"], r["w"],
                            r["group_gap"], case.logits)
    assert mism.size == 0
    gu.check_plan(o, r)
    gu.check_w8a8_out(gu.host_f64(o["out"]), r["out"], gu.w8a8_slack(case), c.name + " layer")


def test_grouped_ffn_w8a8(moe, case):
    c, d = case.cfg, case.device_inputs()
    r = case.ref
    R = int(r["seg_offsets"][-1])
    x_perm, live = gu.x_perm_of(case)
    xq, xs = gu.quantize_act(moe, x_perm)
    so = torch.from_numpy(r["seg_offsets"]).to(gu.dev())
    se = torch.from_numpy(r["seg_expert"]).to(gu.dev())
    q = gu.fp8_weights(moe, d)
    y = gu.empty((moe.moe_num_rows(c), c.H), gu.tdtype(c))
    ws = gu.empty((moe.moe_workspace_size(c),), torch.uint8)
    row_w = gu.row_weights(case)
    moe.moe_grouped_ffn_w8a8(c, xq, xs, so, se, q["w13"], q["w13_s"], q["w2"], q["w2_s"],
                             torch.from_numpy(row_w).to(gu.dev()), y, ws)
    torch.cuda.synchronize()
    ref_s = r["y_perm"][:R] * row_w[:R, None].astype(np.float64)
    # slack of each row: its expert, its token's quantized x, its router weight
    r2t, rows = r["row_to_token"][:R], np.nonzero(live)[0]
    xq64 = ofp8.fake_quant_rows(case.x64)
    slack = np.zeros((R, c.H))
    seg_of_row = np.searchsorted(r["seg_offsets"], np.arange(R), side="right") - 1
    for e in range(c.E):
        sel = rows[r["seg_expert"][seg_of_row[rows]] == e]
        if sel.size:
            slack[sel] = row_w[sel, None] * gu.h_code_slack(xq64[r2t[sel]], case.w13_64[e],
                                                            case.w2_64[e])
    gu.check_w8a8_out(gu.host_f64(y[:R])[live], ref_s[live], slack[live], c.name + " grouped FFN")
