"""Seeded random small layers through moe_layer_forward against the oracle:
shapes, dtypes, routing modes and replica splits drawn at random, so that
every kernel path (fused small-batch routing, multi-kernel permutation,
decode tiles, both ring tile shapes, fp32) meets shapes nobody picked by
hand; and random E4M3-weight layers (some with E4M3 activations too) for
the FP8 tiles, the 64-row short-segment launch among them.  Routing is
compared bit for bit, outputs within the layer tolerance (W8A8: with its
h-code slack rule)."""
import numpy as np
import pytest

import moe_inputs as mi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _random_shape(rng, i):
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    E = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 32, 40, 64]))
    k = int(rng.integers(1, min(E, 6) + 1))
    T = int(rng.choice([1, 2, 7, 33, 64, 100, 257, 600, 1100]))
    # (bf16 sizes in multiples of 8 that are not multiples of the 64-deep
    # stage take the K-tail variants of the ring tiles)
    H = int(rng.choice([64, 128, 192, 320, 512, 1024, 72, 200]))
    I = int(rng.choice([64, 128, 192, 256, 512, 40, 136]))
    if dtype == "f32":
        H = int(rng.choice([4, 12, 64, 100]))
        I = int(rng.choice([3, 16, 70]))
    kw = dict(zipf_s=float(rng.choice([0.0, 1.0, 1.5])))
    if E % 4 == 0 and E >= 8 and rng.random() < 0.4:
        groups = 4
        kw.update(score="sigmoid", n_group=groups, topk_group=int(rng.integers(1, groups + 1)))
        per = E // groups
        k = min(k, kw["topk_group"] * per)
        kw["group_score_topn"] = int(rng.integers(1, min(per, 3) + 1))
    if rng.random() < 0.4 and E >= 2:
        kw.update(n_hot_split=int(rng.integers(1, min(E, 4) + 1)), split_ways=int(rng.integers(2, 4)))
        if rng.random() < 0.5:
            kw.update(split_mode="bounded", split_c_permille=int(rng.choice([0, 100, 700, 2500])))
    elif rng.random() < 0.3:
        kw["capacity_factor_permille"] = int(rng.choice([500, 1000, 1250, 2000]))
    if dtype == "bf16" and rng.random() < 0.2:
        kw["shared_I"] = int(rng.choice([64, 128, 256, 24]))
    if rng.random() < 0.2:
        kw["renormalize"] = 0
    return mi.MoEShape(f"rand{i}", T=T, H=H, E=E, k=k, I=I, dtype=dtype, seed=1000 + i,
                       x_std=0.5, **kw)


@pytest.mark.timeout(600)
def test_random_layers():
    import mixture_experts_layer_segments_amd as moe
    rng = np.random.default_rng(2024)
    for i in range(32):
        cfg = _random_shape(rng, i)
        print(f"\n[random] {i}: {cfg}", flush=True)
        case = gu.SmallCase(cfg)
        o = gu.run_layer(moe, cfg, case.device_inputs())
        r = case.ref
        gu.check_routing(cfg, o["ids"].cpu().numpy(), o["w"].cpu().numpy(), r["ids"], r["w"],
                         r["group_gap"], case.logits)
        gu.check_plan(o, r)
        err = gu.rel_err(gu.host_f64(o["out"]), r["out"])
        assert err <= gu.rel_tol(cfg), (i, err)


def _random_fp8_shape(rng, i):
    """E4M3 weights (and, for about a third of the layers, E4M3 activations)
    on random layers: H and I multiples of 128, segment lengths on both sides
    of the 64-row and 256-row tile boundaries."""
    E = int(rng.choice([2, 3, 8, 12, 16, 32]))
    k = int(rng.integers(1, min(E, 4) + 1))
    T = int(rng.choice([1, 20, 90, 257, 600, 1100]))
    H = int(rng.choice([128, 256, 384]))
    I = int(rng.choice([128, 256]))
    acts = "fp8" if rng.random() < 0.35 else "bf16"
    kw = dict(zipf_s=float(rng.choice([0.0, 1.0, 1.5])))
    if E % 4 == 0 and E >= 8 and rng.random() < 0.4:
        kw.update(score="sigmoid", n_group=4, topk_group=int(rng.integers(2, 5)))
        k = min(k, kw["topk_group"] * (E // 4))
    if rng.random() < 0.3 and E >= 2:
        kw.update(n_hot_split=int(rng.integers(1, min(E, 3) + 1)), split_ways=2)
    elif rng.random() < 0.2:
        kw["capacity_factor_permille"] = int(rng.choice([1000, 1250]))
    if rng.random() < 0.25:
        kw["shared_I"] = int(rng.choice([128, 256]))
    return mi.MoEShape(f"rand8_{i}", T=T, H=H, E=E, k=k, I=I, seed=3000 + i, x_std=0.5,
                       weights="fp8", acts=acts, **kw)


@pytest.mark.timeout(600)
def test_random_fp8_layers():
    import mixture_experts_layer_segments_amd as moe
    rng = np.random.default_rng(2025)
    for i in range(24):
        cfg = _random_fp8_shape(rng, i)
        print(f"\n[random fp8] {i}: {cfg}", flush=True)
        case = gu.SmallCase(cfg)
        o = gu.run_layer(moe, cfg, case.device_inputs())
        r = case.ref
        gu.check_routing(cfg, o["ids"].cpu().numpy(), o["w"].cpu().numpy(), r["ids"], r["w"],
                         r["group_gap"], case.logits)
        gu.check_plan(o, r)
        got = gu.host_f64(o["out"])
        if cfg.acts == "fp8":
            gu.check_w8a8_out(got, r["out"], gu.w8a8_slack(case), cfg.name)
        else:
            err = gu.rel_err(got, r["out"])
            assert err <= gu.rel_tol(cfg), (i, err)
