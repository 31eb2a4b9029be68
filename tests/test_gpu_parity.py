"""GPU parity of every C-ABI call against the CPU oracle on small layers that
the whole oracle finishes in seconds, spanning several tiles with ragged
tails, plus the degenerate cases (one expert, k = E, one hot expert taking
every token, parity and load-bounded replica splits, dropped ids, an empty
batch)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import fp8 as ofp8
from oracle import moe_oracle as orc
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SHAPES = {
    "tiny_fp32": mi.WORKLOADS["tiny_fp32"],
    "bf16_tiles_hot_split": mi.MoEShape("t1", T=300, H=576, E=16, k=4, I=320, zipf_s=1.2,
                                        n_hot_split=3, split_ways=2, seed=11),
    "bf16_grouped_shared": mi.MoEShape("t2", T=200, H=256, E=32, k=4, I=128, score="sigmoid",
                                       n_group=4, topk_group=2, shared_I=192, zipf_s=1.0,
                                       seed=12),
    "f32_ragged": mi.MoEShape("t3", T=50, H=132, E=10, k=3, I=70, dtype="f32", seed=13),
    "bf16_one_expert": mi.MoEShape("t4", T=70, H=128, E=1, k=1, I=64, seed=14),
    "bf16_k_equals_E": mi.MoEShape("t5", T=33, H=192, E=4, k=4, I=128, seed=15),
    "bf16_three_way_split": mi.MoEShape("t6", T=257, H=128, E=12, k=3, I=64, zipf_s=1.5,
                                        n_hot_split=2, split_ways=3, seed=16),
    "bf16_single_token": mi.MoEShape("t7", T=1, H=512, E=64, k=8, I=256, seed=17),
    "bf16_no_renorm_sigmoid": mi.MoEShape("t8", T=90, H=256, E=64, k=6, I=128, score="sigmoid",
                                          n_group=8, topk_group=3, renormalize=0, seed=18),
    "bf16_no_renorm_softmax": mi.MoEShape("t9", T=90, H=256, E=48, k=5, I=128, renormalize=0,
                                          seed=19),
    # few rows per segment and K a multiple of 1024 / 512: the weight-streaming kernels
    "bf16_decode_stream": mi.MoEShape("t10", T=40, H=1024, E=32, k=2, I=512, seed=20),
    "bf16_decode_stream_shared": mi.MoEShape("t11", T=24, H=2048, E=16, k=2, I=512,
                                             score="sigmoid", n_group=4, topk_group=2,
                                             shared_I=1024, seed=24),
    # many rows per segment (256 x 256 tiles), N and K tails in both GEMMs
    "bf16_big_tiles": mi.MoEShape("t12", T=1100, H=320, E=3, k=1, I=192, zipf_s=1.0,
                                  seed=25),
    # load-bounded replica splits: balanced (C = 0), relaxed, and C large enough
    # that replica 0 takes everything; both the one-workgroup path (T*k <= 1024)
    # and the four-kernel permutation
    "bf16_bounded_split": mi.MoEShape("t13", T=300, H=576, E=16, k=4, I=320, zipf_s=1.2,
                                      n_hot_split=3, split_ways=2, split_mode="bounded",
                                      seed=26),
    "bf16_bounded_three_way": mi.MoEShape("t14", T=257, H=128, E=12, k=3, I=64, zipf_s=1.5,
                                          n_hot_split=2, split_ways=3, split_mode="bounded",
                                          split_c_permille=500, seed=27),
    "bf16_bounded_decode": mi.MoEShape("t15", T=40, H=1024, E=32, k=2, I=512, zipf_s=1.0,
                                       n_hot_split=4, split_ways=4, split_mode="bounded",
                                       split_c_permille=250, seed=28),
    "f32_bounded_all_to_first": mi.MoEShape("t16", T=50, H=132, E=10, k=3, I=70, dtype="f32",
                                            zipf_s=1.0, n_hot_split=2, split_ways=4,
                                            split_mode="bounded", split_c_permille=3000,
                                            seed=29),
    # fixed-capacity layout with drops: weight-streaming tiles through the
    # one-workgroup planner, ring tiles through the four-kernel one, fp32, and
    # a capacity that holds every assignment (more slots than assignments)
    "bf16_capacity_decode": mi.MoEShape("t17", T=40, H=1024, E=32, k=2, I=512, zipf_s=1.0,
                                        capacity_factor_permille=1250, seed=30),
    "bf16_capacity_rings": mi.MoEShape("t18", T=300, H=576, E=16, k=4, I=320, zipf_s=1.2,
                                       capacity_factor_permille=1000, seed=31),
    "f32_capacity": mi.MoEShape("t19", T=50, H=132, E=10, k=3, I=70, dtype="f32", zipf_s=1.0,
                                capacity_factor_permille=800, seed=32),
    "bf16_capacity_roomy": mi.MoEShape("t20", T=120, H=256, E=8, k=2, I=128, zipf_s=1.0,
                                       capacity_factor_permille=4000, seed=33),
    # H and I multiples of 8 but not of the 64-deep stage: the last K stage of
    # each GEMM is partial (128-row tiles; 256-row tiles; a single partial
    # stage; a shared expert beside the routed ones)
    "bf16_k_tail_mid": mi.MoEShape("t21", T=300, H=200, E=16, k=4, I=72, zipf_s=1.2, seed=34),
    "bf16_k_tail_big": mi.MoEShape("t22", T=1100, H=264, E=3, k=1, I=136, zipf_s=1.0, seed=35),
    "bf16_k_tail_one_stage": mi.MoEShape("t23", T=64, H=8, E=8, k=2, I=16, seed=36),
    "bf16_k_tail_shared": mi.MoEShape("t24", T=200, H=136, E=32, k=4, I=72, score="sigmoid",
                                      n_group=4, topk_group=2, shared_I=40, zipf_s=1.0,
                                      seed=37),
    # flat routing on 32 lanes per token: inside the one-workgroup planner
    # (T*k <= 1024), and flat sigmoid weights through the four-kernel path
    "bf16_wide_k_small": mi.MoEShape("t25", T=40, H=128, E=64, k=20, I=64, seed=38),
    "bf16_flat_sigmoid_wide": mi.MoEShape("t26", T=60, H=128, E=40, k=18, I=64, score="sigmoid",
                                          seed=39),
    # many bins and segments: 1024 experts with 4-way parity replicas of the 8
    # hottest (4096 bins, 1048 segments) through the four-kernel planner and
    # the one-workgroup one, and a fixed-capacity layout of 2048 segments
    "bf16_many_segments": mi.MoEShape("t27", T=600, H=64, E=1024, k=4, I=64, zipf_s=1.0,
                                      n_hot_split=8, split_ways=4, seed=40),
    "bf16_many_segments_small": mi.MoEShape("t28", T=200, H=64, E=1024, k=4, I=64, zipf_s=1.0,
                                            n_hot_split=8, split_ways=4, seed=41),
    "bf16_capacity_many": mi.MoEShape("t29", T=600, H=64, E=1024, k=2, I=64, zipf_s=1.0,
                                      capacity_factor_permille=1000, seed=42),
    # unsplit dropless layers of 65-256 experts, planned by one wave with 2, 3
    # or 4 experts per lane, through the planning kernel (T*k > 1024) and the
    # one-workgroup kernel (T*k <= 1024; grouped routing on whole waves too)
    "bf16_wave_plan_2": mi.MoEShape("t30", T=300, H=64, E=100, k=4, I=64, zipf_s=1.0, seed=43),
    "bf16_wave_plan_3_small": mi.MoEShape("t31", T=100, H=64, E=160, k=6, I=64, zipf_s=1.0,
                                          seed=44),
    "bf16_wave_plan_4": mi.MoEShape("t32", T=200, H=64, E=256, k=8, I=64, zipf_s=1.0, seed=45),
    "bf16_wave_plan_4_small": mi.MoEShape("t33", T=64, H=64, E=256, k=8, I=64, zipf_s=1.0,
                                          seed=46),
    "bf16_wave_plan_grouped_small": mi.MoEShape("t34", T=50, H=64, E=192, k=6, I=64,
                                                score="sigmoid", n_group=8, topk_group=3,
                                                seed=47),
}


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_segments_amd as m
    return m


@pytest.fixture(scope="module", params=sorted(SHAPES))
def case(request):
    print(f"\n[case] {request.param}", flush=True)
    return gu.SmallCase(SHAPES[request.param])


def test_route(moe, case):
    c, d = case.cfg, case.device_inputs()
    ids = gu.empty((c.T, c.k), torch.int32)
    w = gu.empty((c.T, c.k), torch.float32)
    moe.moe_route_topk(c, d["logits"], ids, w)
    torch.cuda.synchronize()
    mism = gu.check_routing(c, ids.cpu().numpy(), w.cpu().numpy(), case.ref["ids"],
                            case.ref["w"], case.ref["group_gap"], case.logits)
    assert mism.size == 0


def test_permute(moe, case):
    c, d = case.cfg, case.device_inputs()
    ids_d = torch.from_numpy(case.ref["ids"]).to(gu.dev())
    g = gu.run_permute(moe, c, d["x"], ids_d)
    gu.check_plan(g, case.ref)
    R = int(case.ref["seg_offsets"][-1])
    live = torch.from_numpy(case.ref["row_to_token"][:R] >= 0)   # not padding
    xp = g["x_perm"][:R].cpu()[live]
    expect = d["x"].cpu()[torch.from_numpy(case.ref["row_to_token"][:R]).long()[live]]
    assert torch.equal(xp.view(torch.int16) if c.dtype == "bf16" else xp.view(torch.int32),
                       expect.view(torch.int16) if c.dtype == "bf16" else expect.view(torch.int32))


def test_grouped_ffn(moe, case):
    c, d = case.cfg, case.device_inputs()
    r = case.ref
    R = int(r["seg_offsets"][-1])
    x_perm, live = gu.x_perm_of(case)
    so = torch.from_numpy(r["seg_offsets"]).to(gu.dev())
    se = torch.from_numpy(r["seg_expert"]).to(gu.dev())
    y = gu.empty((moe.moe_num_rows(c), c.H), gu.tdtype(c))
    ws = gu.empty((moe.moe_workspace_size(c),), torch.uint8)
    moe.moe_grouped_ffn(c, x_perm, so, se, d["w13"], d["w2"], None, y, ws)
    torch.cuda.synchronize()
    err = gu.rel_err(gu.host_f64(y[:R])[live], r["y_perm"][:R][live])
    assert err <= gu.rel_tol(c), err
    # router weight applied in the epilogue
    row_w = gu.row_weights(case)
    moe.moe_grouped_ffn(c, x_perm, so, se, d["w13"], d["w2"],
                        torch.from_numpy(row_w).to(gu.dev()), y, ws)
    torch.cuda.synchronize()
    ref_s = r["y_perm"][:R] * row_w[:R, None].astype(np.float64)
    err = gu.rel_err(gu.host_f64(y[:R])[live], ref_s[live])
    assert err <= gu.rel_tol(c), err


def test_combine(moe, case):
    c, d = case.cfg, case.device_inputs()
    r = case.ref
    y_enc = mi.bf16_bits(r["y_perm"].astype(np.float32)) if c.dtype == "bf16" \
        else r["y_perm"].astype(np.float32)
    y_in = mi.values_f64(y_enc, c.dtype)
    sh_enc = sh_in = None
    if r["shared_y"] is not None:
        sh_enc = mi.bf16_bits(r["shared_y"].astype(np.float32)) if c.dtype == "bf16" \
            else r["shared_y"].astype(np.float32)
        sh_in = mi.values_f64(sh_enc, c.dtype)
    out = gu.empty((c.T, c.H), gu.tdtype(c))
    w32 = r["w"].astype(np.float32)
    moe.moe_unpermute_combine(c, gu.to_dev(y_enc, c.dtype),
                              torch.from_numpy(r["assign_to_row"]).to(gu.dev()),
                              torch.from_numpy(w32).to(gu.dev()),
                              None if sh_enc is None else gu.to_dev(sh_enc, c.dtype), out)
    torch.cuda.synchronize()
    ref = orc.combine(y_in, r["assign_to_row"], w32.astype(np.float64), sh_in)
    # fp32 accumulation of k + 1 terms, one final rounding to the output type
    tol = (2.0 ** -8 if c.dtype == "bf16" else 2.0 ** -20) * np.abs(ref).max()
    assert np.abs(gu.host_f64(out) - ref).max() <= tol


def test_layer_forward(moe, case):
    c, d = case.cfg, case.device_inputs()
    o = gu.run_layer(moe, c, d)
    r = case.ref
    gu.check_routing(c, o["ids"].cpu().numpy(), o["w"].cpu().numpy(), r["ids"], r["w"],
                     r["group_gap"], case.logits)
    # the layer's own permutation (one workgroup for T*k <= 1024, else the
    # four-kernel path), bit for bit
    gu.check_plan(o, r)
    err = gu.rel_err(gu.host_f64(o["out"]), r["out"])
    print(f"  layer rel err {err:.3e}")
    assert err <= gu.rel_tol(c), err
    # deterministic: a second run is bit-identical
    o2 = gu.run_layer(moe, c, d)
    assert torch.equal(o["out"].view(torch.int16) if c.dtype == "bf16" else o["out"],
                       o2["out"].view(torch.int16) if c.dtype == "bf16" else o2["out"])


def test_one_hot_expert_takes_every_token(moe):
    """Every token routes first to expert 5: one segment holds every slot-0
    row and most segments are empty."""
    cfg = mi.MoEShape("hot", T=333, H=256, E=16, k=2, I=128, seed=21)
    lg = mi.logits(cfg)
    lg[:, 5] = lg.max(axis=1) + 1.0
    case = gu.SmallCase(cfg, logits=lg)
    o = gu.run_layer(moe, cfg, case.device_inputs())
    assert o["counts"].cpu().numpy()[5] == cfg.T
    assert (o["counts"].cpu().numpy() == case.ref["counts"]).all()
    assert o["bal"].cpu().numpy()[0] == case.ref["balancedness"]
    assert gu.rel_err(gu.host_f64(o["out"]), case.ref["out"]) <= gu.BF16_REL


@pytest.mark.parametrize("split_mode", ["parity", "bounded", "capacity"])
def test_dropped_ids(moe, split_mode):
    """Ids outside [0, E) join no segment and get assign_to_row = -1."""
    if split_mode == "capacity":
        cfg = mi.MoEShape("drop", T=40, H=128, E=6, k=3, I=64, capacity_factor_permille=900,
                          seed=22)
    else:
        cfg = mi.MoEShape("drop", T=40, H=128, E=6, k=3, I=64, n_hot_split=1, split_ways=2,
                          split_mode=split_mode, split_c_permille=200, seed=22)
    rng = np.random.default_rng(0)
    ids = rng.integers(0, cfg.E, size=(cfg.T, cfg.k)).astype(np.int32)
    bad = rng.random((cfg.T, cfg.k)) < 0.2
    ids[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, cfg.E)
    x = mi.x(cfg)
    g = gu.run_permute(moe, cfg, gu.to_dev(x, cfg.dtype), torch.from_numpy(ids).to(gu.dev()))
    valid = ~bad.ravel()
    counts = np.bincount(ids.ravel()[valid], minlength=cfg.E)
    if split_mode == "capacity":
        p = orc.capacity_plan(ids, cfg.E, orc.capacity(ids.size, cfg.E, 900))
        p.update(counts=counts, balancedness=orc.balancedness(counts))
        gu.check_plan(g, p)
        return
    se, sr = orc.segment_list(counts, cfg.n_hot_split, cfg.split_ways)
    if split_mode == "parity":
        seg = orc.segment_of_assignments(np.where(bad, 0, ids), se, sr, cfg.split_ways)
    else:
        # the valid assignments alone, in increasing a, as one column
        loads = {int(e): orc.replica_loads(int(counts[e]), cfg.split_ways, cfg.split_c_permille)
                 for e in set(se[sr >= 0].tolist())}
        seg = np.zeros(ids.size, dtype=np.int64)
        seg[valid] = orc.segment_of_assignments(ids.ravel()[valid][:, None], se, sr,
                                                cfg.split_ways, loads)
    seg = np.where(valid, seg, len(se))   # dropped -> a sentinel past the end
    so, r2a, a2r, r2t = orc.permutation(seg, len(se) + 1, cfg.k)
    a2r = np.where(valid, a2r, -1)
    assert (g["counts"].cpu().numpy() == counts).all()
    assert (g["seg_offsets"].cpu().numpy() == so[:len(se) + 1]).all()
    assert (g["a2r"].cpu().numpy() == a2r).all()
    R = int(so[len(se)])
    assert (g["r2t"].cpu().numpy()[:R] == r2t[:R]).all()
    assert g["bal"].cpu().numpy()[0] == orc.balancedness(counts)


# flat routing runs on 16 lanes per token (k <= 16, E <= 256), 32 lanes
# (k <= 32, E <= 512) or a whole wave; k equal to the group width, and 1 or 16
# logits per lane, included
@pytest.mark.parametrize("E,k,groups,topk_group", [(1024, 32, 1, 1), (100, 7, 1, 1),
                                                   (256, 8, 64, 16), (130, 3, 1, 1),
                                                   (512, 20, 1, 1), (300, 16, 1, 1),
                                                   (16, 16, 1, 1), (64, 32, 1, 1)])
def test_route_extremes(moe, E, k, groups, topk_group):
    score = "sigmoid" if groups > 1 else "softmax"
    cfg = mi.MoEShape("rx", T=77, H=64, E=E, k=k, I=64, score=score, n_group=groups,
                      topk_group=topk_group, seed=23)
    lg = mi.logits(cfg)
    ids_r, w_r, gap = orc.route(cfg, lg)
    ids = gu.empty((cfg.T, cfg.k), torch.int32)
    w = gu.empty((cfg.T, cfg.k), torch.float32)
    moe.moe_route_topk(cfg, torch.from_numpy(lg).to(gu.dev()), ids, w)
    torch.cuda.synchronize()
    gu.check_routing(cfg, ids.cpu().numpy(), w.cpu().numpy(), ids_r, w_r, gap, lg)


# exact ties (values on a 1/2 grid), zeros of both signs (they tie) and -inf
# entries, through every routing path: 16 and 32 lanes per token, the whole
# wave, groups that are lane blocks and groups that are not (12 experts)
@pytest.mark.parametrize("E,k,groups,topk_group", [(128, 8, 1, 1), (512, 20, 1, 1),
                                                   (1024, 32, 1, 1), (256, 8, 8, 4),
                                                   (96, 6, 8, 3), (128, 4, 64, 8)])
def test_route_ties_and_signed_zeros(moe, E, k, groups, topk_group):
    score = "sigmoid" if groups > 1 else "softmax"
    cfg = mi.MoEShape("rt", T=300, H=64, E=E, k=k, I=64, score=score, n_group=groups,
                      topk_group=topk_group, seed=29)
    lg = mi.tied_logits(cfg)
    ids_r, w_r, gap = orc.route(cfg, lg)
    ids = gu.empty((cfg.T, cfg.k), torch.int32)
    w = gu.empty((cfg.T, cfg.k), torch.float32)
    moe.moe_route_topk(cfg, torch.from_numpy(lg).to(gu.dev()), ids, w)
    torch.cuda.synchronize()
    gu.check_routing(cfg, ids.cpu().numpy(), w.cpu().numpy(), ids_r, w_r, gap, lg)


def test_empty_batch_is_a_noop(moe):
    cfg = mi.MoEShape("empty", T=0, H=128, E=8, k=2, I=64)
    sentinel = torch.full((4,), 7, dtype=torch.int32, device=gu.dev())
    moe.moe_route_topk(cfg, None, sentinel, None)
    torch.cuda.synchronize()
    assert (sentinel.cpu() == 7).all()


@pytest.mark.parametrize("T,k,E,n_ids", [(100, 4, 4, 1), (150, 4, 4, 2)])
def test_repeated_ids_make_segments_longer_than_the_batch(moe, T, k, E, n_ids):
    """moe_permute takes ids that repeat within a token, so a segment may hold
    more rows than there are tokens (all ids 0: one segment of T*k rows).
    moe_grouped_ffn on that permutation must compute every row, also when
    the segment reaches the 256-row tiles while T is below 256."""
    cfg = mi.MoEShape("rep", T=T, H=256, E=E, k=k, I=128, seed=34)
    rng = np.random.default_rng(T)
    ids = rng.integers(0, n_ids, size=(T, k)).astype(np.int32)
    x = mi.x(cfg)
    w13b = np.stack([mi.w13(cfg, e) for e in range(E)])
    w2b = np.stack([mi.w2(cfg, e) for e in range(E)])
    g = gu.run_permute(moe, cfg, gu.to_dev(x, cfg.dtype), torch.from_numpy(ids).to(gu.dev()))
    counts = orc.expert_counts(ids, E)
    assert counts.max() > T
    se, sr = orc.segment_list(counts, 0, 1)
    seg = orc.segment_of_assignments(ids, se, sr, 1)
    so, r2a, a2r, r2t = orc.permutation(seg, len(se), k)
    p = dict(counts=counts, seg_offsets=so, seg_expert=se, assign_to_row=a2r,
             row_to_token=r2t, balancedness=orc.balancedness(counts))
    gu.check_plan(g, p)
    y = gu.empty((T * k, cfg.H), torch.bfloat16)
    y.fill_(0)
    ws = gu.empty((moe.moe_workspace_size(cfg),), torch.uint8)
    moe.moe_grouped_ffn(cfg, g["x_perm"], g["seg_offsets"], g["seg_expert"],
                        gu.to_dev(w13b, "bf16"), gu.to_dev(w2b, "bf16"), None, y, ws)
    torch.cuda.synchronize()
    x64 = mi.values_f64(x, "bf16")
    ref = orc.grouped_ffn(x64[r2t], so, se, mi.values_f64(w13b, "bf16"),
                          mi.values_f64(w2b, "bf16"))
    got = gu.host_f64(y)
    err = gu.rel_err(got, ref)
    print(f"  longest segment {counts.max()} rows of {T} tokens: rel err {err:.3e}")
    assert err <= gu.BF16_REL, err
    # every row was written (a skipped segment would leave the zero fill)
    assert (np.abs(got).max(axis=1) > 0).all()


# Segment lengths whose last row tile ends on each side of the 64-row wave
# blocks of the 128-row tiles (lengths under 256) and of the 256-row tiles:
# a wave whose rows all lie past the segment's end skips its MFMAs, the
# others compute.  Each expert holds one segment; the total is above 256,
# so both tile launches run.
WAVE_EDGE_LENS = [1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255,
                  257, 319, 320, 321, 384, 385, 448, 449, 511, 512]


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
def test_last_row_tile_wave_edges(moe, weights):
    """moe_grouped_ffn (bf16 or FP8 weights) on segments of WAVE_EDGE_LENS
    rows: every row of every segment against the oracle's expert MLP."""
    lens = np.array(WAVE_EDGE_LENS, dtype=np.int64)
    E, R = len(lens), int(lens.sum())
    cfg = mi.MoEShape("edges", T=R, H=256, E=E, k=1, I=256, seed=37, weights=weights)
    so = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    se = np.arange(E, dtype=np.int32)
    x = mi.x(cfg)
    w13b = np.stack([mi.w13(cfg, e) for e in range(E)])
    w2b = np.stack([mi.w2(cfg, e) for e in range(E)])
    w13_64, w2_64 = mi.values_f64(w13b, "bf16"), mi.values_f64(w2b, "bf16")
    d13, d2 = gu.to_dev(w13b, "bf16"), gu.to_dev(w2b, "bf16")
    y = gu.empty((R, cfg.H), torch.bfloat16)
    y.fill_(0)
    ws = gu.empty((moe.moe_workspace_size(cfg),), torch.uint8)
    so_d, se_d = torch.from_numpy(so).to(gu.dev()), torch.from_numpy(se).to(gu.dev())
    if weights == "fp8":
        # the oracle runs on its own quantization of the same weights
        w13_64 = np.stack([ofp8.dequantize_blocks(*ofp8.quantize_blocks(m)) for m in w13_64])
        w2_64 = np.stack([ofp8.dequantize_blocks(*ofp8.quantize_blocks(m)) for m in w2_64])
        q13, s13 = gu.quantize_fp8(moe, d13)
        q2, s2 = gu.quantize_fp8(moe, d2)
        moe.moe_grouped_ffn_fp8w(cfg, gu.to_dev(x, "bf16"), so_d, se_d, q13, s13, q2, s2, None,
                                 y, ws)
    else:
        moe.moe_grouped_ffn(cfg, gu.to_dev(x, "bf16"), so_d, se_d, d13, d2, None, y, ws)
    torch.cuda.synchronize()
    ref = orc.grouped_ffn(mi.values_f64(x, "bf16"), so, se, w13_64, w2_64)
    got = gu.host_f64(y)
    for s in range(E):
        r0, r1 = so[s], so[s + 1]
        err = gu.rel_err(got[r0:r1], ref[r0:r1])
        assert err <= gu.BF16_REL, (weights, int(lens[s]), err)
    print(f"  {weights}: {E} segments, rel err {gu.rel_err(got, ref):.3e}")


@pytest.mark.parametrize("T", [40, 400])
def test_every_id_dropped(moe, T):
    """Every id outside [0, E): no row in any segment, every assign_to_row
    -1, zero counts, and balancedness 0 (the oracle's reading of 0/0)."""
    cfg = mi.MoEShape("alldrop", T=T, H=128, E=6, k=3, I=64, seed=35)
    ids = np.where(np.arange(T * cfg.k).reshape(T, cfg.k) % 2 == 0, -1, cfg.E).astype(np.int32)
    g = gu.run_permute(moe, cfg, gu.to_dev(mi.x(cfg), cfg.dtype),
                       torch.from_numpy(ids).to(gu.dev()))
    counts = np.zeros(cfg.E, dtype=np.int64)
    assert (g["counts"].cpu().numpy() == counts).all()
    assert (g["seg_offsets"].cpu().numpy() == 0).all()
    assert (g["a2r"].cpu().numpy() == -1).all()
    assert g["bal"].cpu().numpy()[0] == orc.balancedness(counts)
