"""The whole layer captured once into a HIP graph and replayed on new inputs.

The MoE inference blog ("Prefill and decode kernel layouts") pads decode
tokens into fixed-size layouts so that one captured graph can be replayed.
Here every launch of moe_layer_forward has a grid that depends only on the
configuration: segment lengths and tile tables are built on the device from
the routed ids.  So one graph, captured once, serves batches whose routing
(and so every segment length) differs from the captured one, in the packed
layout and in the fixed-capacity one.  Each replay runs after new logits and
activations are copied into the captured input buffers (eager work between
replays), and its outputs are compared bit for bit with an eager call on the
same inputs; the last replay is also compared with the oracle.
"""
import pytest
import torch

import moe_inputs as mi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = {
    "decode": mi.MoEShape("g1", T=64, H=1024, E=32, k=2, I=512, zipf_s=1.0, seed=41),
    "decode_capacity": mi.MoEShape("g2", T=64, H=1024, E=32, k=2, I=512, zipf_s=1.0,
                                   capacity_factor_permille=1250, seed=42),
    # T*k > 1024: the four-kernel permutation and the ring tiles
    "rings_grouped_shared": mi.MoEShape("g3", T=300, H=256, E=32, k=4, I=128,
                                        score="sigmoid", n_group=4, topk_group=2,
                                        shared_I=256, zipf_s=1.0, seed=43),
    "decode_fp8": mi.MoEShape("g4", T=64, H=1024, E=32, k=2, I=512, zipf_s=1.0,
                              weights="fp8", seed=44),
    # E4M3 weights on the ring tiles; E4M3 activations too, on the decode
    # tiles (x and h quantized between launches) and on the ring tiles (h
    # quantized in GEMM 1's epilogue)
    "rings_fp8": mi.MoEShape("g5", T=300, H=256, E=32, k=4, I=128, zipf_s=1.0,
                             weights="fp8", seed=45),
    "decode_w8a8": mi.MoEShape("g6", T=64, H=1024, E=32, k=2, I=512, zipf_s=1.0,
                               weights="fp8", acts="fp8", seed=46),
    "rings_w8a8": mi.MoEShape("g7", T=300, H=256, E=32, k=4, I=128, zipf_s=1.0,
                              weights="fp8", acts="fp8", seed=47),
}


class Layer:
    """Outputs, workspace and the call of one layer configuration."""

    def __init__(self, moe, cfg, d):
        self.moe, self.cfg, self.d = moe, cfg, d
        tdt = gu.tdtype(cfg)
        self.o = dict(out=gu.empty((cfg.T, cfg.H), tdt),
                      ids=gu.empty((cfg.T, cfg.k), torch.int32),
                      w=gu.empty((cfg.T, cfg.k), torch.float32),
                      counts=gu.empty((cfg.E,), torch.int32), bal=gu.empty((1,), torch.float32))
        self.ws = gu.empty((moe.moe_workspace_size(cfg),), torch.uint8)

    def __call__(self):
        d, o, m = self.d, self.o, self.moe
        if self.cfg.weights == "fp8":
            call = m.moe_layer_forward_w8a8 if self.cfg.acts == "fp8" else m.moe_layer_forward_fp8w
            call(self.cfg, d["logits"], d["x"], d["w13"], d["w13_s"], d["w2"], d["w2_s"],
                 d["sw13"], d["sw13_s"], d["sw2"], d["sw2_s"], o["out"], o["ids"], o["w"],
                 o["counts"], o["bal"], self.ws)
        else:
            m.moe_layer_forward(self.cfg, d["logits"], d["x"], d["w13"], d["w2"], d["sw13"],
                                d["sw2"], o["out"], o["ids"], o["w"], o["counts"], o["bal"],
                                self.ws)

    def snapshot(self):
        return {k: v.clone() for k, v in self.o.items()}


def _same(a, b):
    for k in a:
        x, y = a[k], b[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), k


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replay_matches_eager(name):
    import mixture_experts_layer_segments_amd as moe
    cfg = CASES[name]
    print(f"\n[graph] {name}: inputs", flush=True)
    case = gu.SmallCase(cfg)
    d = case.device_inputs()
    if cfg.weights == "fp8":
        d = gu.fp8_weights(moe, d)
    layer = Layer(moe, cfg, d)
    eager = Layer(moe, cfg, d)           # own outputs and workspace, same inputs

    # warm up on a side stream (first calls query the device), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    torch.cuda.synchronize()
    print(f"[graph] {name}: captured", flush=True)

    seeds = [cfg.seed + 100, cfg.seed + 200, cfg.seed]
    for it, seed in enumerate(seeds):
        other = cfg.replace(seed=seed)
        lg, xb = mi.logits(other), mi.x(other)
        d["logits"].copy_(torch.from_numpy(lg))
        d["x"].copy_(gu.to_dev(xb, cfg.dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = layer.snapshot()
        eager()
        torch.cuda.synchronize()
        _same(got, eager.snapshot())
        print(f"[graph] {name}: replay {it} (seed {seed}) equals eager, counts "
              f"{got['counts'].cpu().numpy().tolist()[:8]}...", flush=True)
    # the last inputs are the case's own: the replay also matches the oracle
    r = case.ref
    mism = gu.check_routing(cfg, got["ids"].cpu().numpy(), got["w"].cpu().numpy(), r["ids"],
                            r["w"], r["group_gap"], case.logits)
    assert mism.size == 0
    assert (got["counts"].cpu().numpy() == r["counts"]).all()
    if cfg.acts == "fp8":
        gu.check_w8a8_out(gu.host_f64(got["out"]), r["out"], gu.w8a8_slack(case),
                          f"[graph] {name}: last replay vs oracle")
        return
    err = gu.rel_err(gu.host_f64(got["out"]), r["out"])
    print(f"[graph] {name}: last replay vs oracle rel err {err:.3e}", flush=True)
    assert err <= gu.rel_tol(cfg), err
