"""GPU parity of the FP8-weight path against the oracle.

* moe_quantize_fp8: codes and scales bit for bit against the oracle's own
  block quantizer -- on random matrices spanning many scales (zero blocks,
  subnormal-range elements, negative zeros) and on every finite bf16 value
  in [-448, 448] at scale 1.
* moe_layer_forward_fp8w / moe_grouped_ffn_fp8w on small layers that span
  both GEMM families (weight-streaming decode tiles, 128 x 256 and 256 x 256
  ring tiles) with shared experts, groups and replica splits: routing bit for
  bit, outputs within the bf16 layer tolerance of the oracle run on the
  oracle's dequantized weights (the dequantized values are exact in bf16, so
  the kernels multiply exactly those numbers).
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import fp8 as ofp8
from oracle import moe_oracle as orc
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_segments_amd as m
    return m


def _bf16_bits(values_f32: np.ndarray) -> np.ndarray:
    return mi.bf16_bits(values_f32.astype(np.float32))


def _check_codes(moe, bits: np.ndarray):
    """bits: bf16 bit patterns [n, R, C] -> compare the library's codes and
    scales with the oracle's, exactly."""
    src = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(gu.dev()).view(torch.bfloat16)
    q, sc = gu.quantize_fp8(moe, src)
    torch.cuda.synchronize()
    vals = mi.values_f64(bits, "bf16")
    for m in range(bits.shape[0]):
        c_ref, s_ref = ofp8.quantize_blocks(vals[m])
        c_got = q[m].cpu().numpy()
        bad = np.argwhere(c_got != c_ref)
        assert bad.size == 0, (m, bad[:5], c_got[tuple(bad[0])], c_ref[tuple(bad[0])],
                               vals[m][tuple(bad[0])])
        assert np.array_equal(sc[m].cpu().numpy().astype(np.float64), s_ref), m


def test_quantizer_random_scales(moe):
    rng = np.random.default_rng(21)
    w = rng.normal(0, 1.0, size=(3, 256, 384))
    blk_scale = 2.0 ** rng.integers(-30, 30, size=(3, 2, 3))
    w *= np.repeat(np.repeat(blk_scale, 128, axis=1), 128, axis=2)
    w[0, :128, :128] = 0.0                                  # all-zero block
    w[1, 128:, 256:] *= np.where(rng.random((128, 128)) < 0.5, 2.0 ** -12, 1.0)  # subnormal range
    w[2, 5, 7] = -0.0
    w[2, 0:128, 0:128] = np.round(w[2, 0:128, 0:128] * 4) / 4   # many exact ties after scaling
    _check_codes(moe, _bf16_bits(w))


def test_quantizer_every_bf16_in_range(moe):
    pos = np.arange(0, 0x43E1, dtype=np.uint32)              # +0 .. 448 (0x43E0)
    allv = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    n_blk = -(-allv.size // (128 * 128 - 1))
    flat = np.zeros((n_blk, 128 * 128), dtype=np.uint16)
    for b in range(n_blk):
        chunk = allv[b * (128 * 128 - 1):(b + 1) * (128 * 128 - 1)]
        flat[b, 0] = 0x43E0                                   # 448: every block has scale 1
        flat[b, 1:1 + chunk.size] = chunk
    bits = flat.reshape(n_blk, 128, 128)
    _check_codes(moe, bits)


SHAPES = {
    # weight-streaming decode tiles (K multiples of 256)
    "fp8_decode": mi.MoEShape("f1", T=40, H=1024, E=32, k=2, I=512, weights="fp8", seed=31),
    "fp8_decode_shared_grouped": mi.MoEShape("f2", T=24, H=2048, E=16, k=2, I=512,
                                             score="sigmoid", n_group=4, topk_group=2,
                                             shared_I=1024, weights="fp8", seed=32),
    # 128 x 256 ring tiles with replica splits and N / K tails of the tiles
    "fp8_mid_split": mi.MoEShape("f3", T=300, H=640, E=16, k=4, I=384, zipf_s=1.2,
                                 n_hot_split=3, split_ways=2, weights="fp8", seed=33),
    # 256 x 256 ring tiles (segments of 256 rows and more)
    "fp8_big": mi.MoEShape("f4", T=1100, H=384, E=3, k=1, I=256, zipf_s=1.0, weights="fp8",
                           seed=34),
    # ring tiles with groups and a shared expert
    "fp8_grouped_shared": mi.MoEShape("f5", T=200, H=256, E=32, k=4, I=128, score="sigmoid",
                                      n_group=4, topk_group=2, shared_I=256, zipf_s=1.0,
                                      weights="fp8", seed=35),
    # fixed-capacity layout with drops
    "fp8_capacity": mi.MoEShape("f6", T=40, H=1024, E=32, k=2, I=512, zipf_s=1.0,
                                capacity_factor_permille=1250, weights="fp8", seed=36),
}


@pytest.fixture(scope="module", params=sorted(SHAPES))
def case(request):
    print(f"\n[fp8 case] {request.param}", flush=True)
    return gu.SmallCase(SHAPES[request.param])


def test_layer_forward_fp8(moe, case):
    c = case.cfg
    o = gu.run_layer(moe, c, case.device_inputs())
    for name, (codes, scales) in case.q.items():
        got = o["q"][name]
        got = got if got.dim() == 3 else got[None]
        assert np.array_equal(got.cpu().numpy(), codes), name
        gs = o["q"][name + "_s"]
        gs = gs if gs.dim() == 3 else gs[None]
        assert np.array_equal(gs.cpu().numpy().astype(np.float64), scales), name
    r = case.ref
    mism = gu.check_routing(c, o["ids"].cpu().numpy(), o["w"].cpu().numpy(), r["ids"], r["w"],
                            r["group_gap"], case.logits)
    assert mism.size == 0
    err = gu.rel_err(gu.host_f64(o["out"]), r["out"])
    print(f"[fp8 case] {c.name}: layer rel err {err:.3e}", flush=True)
    assert err <= gu.BF16_REL, err


def test_grouped_ffn_fp8(moe, case):
    c, d = case.cfg, case.device_inputs()
    r = case.ref
    R = int(r["seg_offsets"][-1])
    x_perm, live = gu.x_perm_of(case)
    so = torch.from_numpy(r["seg_offsets"]).to(gu.dev())
    se = torch.from_numpy(r["seg_expert"]).to(gu.dev())
    q = gu.fp8_weights(moe, d)
    y = gu.empty((moe.moe_num_rows(c), c.H), gu.tdtype(c))
    ws = gu.empty((moe.moe_workspace_size(c),), torch.uint8)
    moe.moe_grouped_ffn_fp8w(c, x_perm, so, se, q["w13"], q["w13_s"], q["w2"], q["w2_s"], None,
                             y, ws)
    torch.cuda.synchronize()
    err = gu.rel_err(gu.host_f64(y[:R])[live], r["y_perm"][:R][live])
    print(f"[fp8 case] {c.name}: grouped FFN rel err {err:.3e}", flush=True)
    assert err <= gu.BF16_REL, err
    # router weight applied in the epilogue
    row_w = gu.row_weights(case)
    moe.moe_grouped_ffn_fp8w(c, x_perm, so, se, q["w13"], q["w13_s"], q["w2"], q["w2_s"],
                             torch.from_numpy(row_w).to(gu.dev()), y, ws)
    torch.cuda.synchronize()
    ref_s = r["y_perm"][:R] * row_w[:R, None].astype(np.float64)
    err = gu.rel_err(gu.host_f64(y[:R])[live], ref_s[live])
    assert err <= gu.BF16_REL, err
