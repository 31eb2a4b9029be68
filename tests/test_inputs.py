"""The seeded input generator: encodings and the workloads' stated structure."""
import numpy as np
import torch

import moe_inputs as mi
from oracle import moe_oracle as o


def test_bf16_encoding_is_round_to_nearest_even():
    """The generator's fp32 -> bf16 encoding agrees with torch's conversion
    (round to nearest, ties to even) on random and on tie cases."""
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 3,
        # exact ties: low 16 bits = 0x8000, with odd and even upper halves
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -2.5, 3.0e38, 1e-40], dtype=np.float32),
    ])
    ours = mi.bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    back = mi.bf16_to_f32(ours)
    assert (back == torch.from_numpy(a).to(torch.bfloat16).float().numpy()).all()


def test_logits_rows_are_distinct_and_seeded():
    for name in ["tiny_fp32", "decode_bf16", "deepseek_v3_bf16"]:
        cfg = mi.WORKLOADS[name]
        a = mi.logits(cfg)
        assert a.dtype == np.float32 and a.shape == (cfg.T, cfg.E)
        s = np.sort(a, axis=1)
        assert not (s[:, 1:] == s[:, :-1]).any()
        assert (a == mi.logits(cfg)).all()


def test_workload_structure_matches_its_description():
    """Prefill: balancedness about 0.4-0.5; ragged stress: many empty and tiny
    segments next to very large ones; decode: near-uniform expected load."""
    c3 = mi.WORKLOADS["prefill_skew_bf16"]
    ids, _, _ = o.route(c3, mi.logits(c3))
    b = float(o.balancedness(o.expert_counts(ids, c3.E)))
    assert 0.38 <= b <= 0.55, b
    c5 = mi.WORKLOADS["ragged_stress_bf16"]
    ids, _, _ = o.route(c5, mi.logits(c5))
    p = o.plan(c5, ids)
    lens = np.diff(p["seg_offsets"])
    assert len(lens) == 136
    assert (lens == 0).sum() >= 10 and (lens < 16).sum() >= 40 and lens.max() > 4000
    c2 = mi.WORKLOADS["decode_bf16"]
    ids, _, _ = o.route(c2, mi.logits(c2))
    assert 40 <= (o.expert_counts(ids, c2.E) > 0).sum() <= 64


def test_weights_are_per_expert_streams():
    cfg = mi.WORKLOADS["tiny_fp32"]
    a, b = mi.w13(cfg, 3), mi.w13(cfg, 4)
    assert a.shape == (2 * cfg.I, cfg.H) and not (a == b).all()
    assert (a == mi.w13(cfg, 3)).all()
    assert abs(float(np.std(a)) - 0.02) < 0.001
    bf = mi.WORKLOADS["decode_bf16"].replace(H=64, I=32, E=2)
    w = mi.w2(bf, 1)
    assert w.dtype == np.uint16 and w.shape == (64, 32)
