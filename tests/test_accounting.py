"""The benchmark's byte and flop accounting against the figures the book
prints ("Serving Mixture-of-Experts Models", section "Price one dispatch")."""
import json
import os

import bench
import moe_inputs as mi

GOLD = os.path.join(os.path.dirname(__file__), "golden", "serving_moe_token_flow.json")


def test_dispatch_bytes_match_the_printed_examples():
    with open(GOLD) as f:
        cases = json.load(f)["dispatch"]
    for c in cases:
        cfg = mi.WORKLOADS["decode_bf16"].replace(T=c["tokens"], k=c["top_k"], H=c["hidden"])
        assert cfg.A == c["assignments"]
        assert bench.dispatch_bytes(cfg) == c["bytes"]
        assert bench.dispatch_bytes(cfg, 1) == c["bytes_per_assignment"]
    # the two printed cases are exactly the decode and prefill workloads
    assert bench.dispatch_bytes(mi.WORKLOADS["decode_bf16"]) == 2 * 2 ** 20
    assert bench.dispatch_bytes(mi.WORKLOADS["prefill_skew_bf16"]) == 125 * 2 ** 20


def test_ffn_flops_and_bytes():
    cfg = mi.WORKLOADS["decode_bf16"]
    # 6 H I flops per assignment: gate, up and down projections
    assert bench.ffn_flops(cfg) == 6 * 8192 * 2048 * 128
    # 55 active experts' weights once plus x_perm, h (twice) and y_perm rows
    assert bench.ffn_bytes(cfg, 55) == 55 * 3 * 8192 * 2048 * 2 + 128 * (2 * 8192 + 2 * 2048) * 2
    ds = mi.WORKLOADS["deepseek_v3_bf16"]
    assert bench.ffn_flops(ds) - bench.ffn_flops(ds.replace(shared_I=0)) == 6 * 7168 * 2048 * 4096
