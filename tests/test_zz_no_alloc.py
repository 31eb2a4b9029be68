"""moe_layer_forward_static, the entry point that allocates nothing (its
workspace is a device array inside the library), against moe_layer_forward
on a caller workspace: two calls in a row, the second with a smaller batch,
each bit for bit equal to moe_layer_forward and within tolerance of the
oracle; and a layer too large for the array is refused before any launch."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_segments_amd as m
    return m


def _outputs(cfg):
    return dict(out=gu.empty((cfg.T, cfg.H), gu.tdtype(cfg)),
                ids=gu.empty((cfg.T, cfg.k), torch.int32),
                w=gu.empty((cfg.T, cfg.k), torch.float32),
                counts=gu.empty((cfg.E,), torch.int32), bal=gu.empty((1,), torch.float32))


def _static_layer(moe, cfg, d):
    o = _outputs(cfg)
    moe.moe_layer_forward_static(cfg, d["logits"], d["x"], d["w13"], d["w2"], d["sw13"],
                                 d["sw2"], o["out"], o["ids"], o["w"], o["counts"], o["bal"])
    torch.cuda.synchronize()
    return o


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


# the decode layer (weight-streaming tiles, one-workgroup planner), then a
# smaller ring-tile layer with groups and a shared expert (four-kernel
# planner), then the tiny decode batch again
SEQUENCE = [
    mi.MoEShape("s1", T=64, H=2048, E=32, k=2, I=512, zipf_s=1.0, seed=61),
    mi.MoEShape("s2", T=40, H=256, E=16, k=4, I=128, score="sigmoid", n_group=4,
                topk_group=2, shared_I=128, zipf_s=1.0, seed=62),
    mi.MoEShape("s3", T=300, H=576, E=16, k=4, I=320, zipf_s=1.2, n_hot_split=3,
                split_ways=2, seed=63),
    mi.MoEShape("s4", T=9, H=256, E=8, k=2, I=128, seed=64),
]


def test_static_workspace_matches_caller_workspace(moe):
    for i, cfg in enumerate(SEQUENCE):
        print(f"\n[no-alloc] call {i}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}", flush=True)
        assert moe.moe_workspace_size(cfg) <= moe.MOE_STATIC_WORKSPACE_BYTES
        case = gu.SmallCase(cfg)
        d = case.device_inputs()
        got = _static_layer(moe, cfg, d)
        ref = gu.run_layer(moe, cfg, d)
        for key in ("out", "ids", "w", "counts", "bal"):
            assert _same(got[key], ref[key]), (i, key)
        err = gu.rel_err(gu.host_f64(got["out"]), case.ref["out"])
        print(f"  bit-equal to moe_layer_forward; rel err vs oracle {err:.3e}", flush=True)
        assert err <= gu.rel_tol(cfg), err
        assert (got["ids"].cpu().numpy() == case.ref["ids"]).all()


def test_too_large_for_the_static_workspace_is_refused(moe):
    cfg = mi.WORKLOADS["prefill_skew_bf16"]
    assert moe.moe_workspace_size(cfg) > moe.MOE_STATIC_WORKSPACE_BYTES
    sentinel = torch.full((4,), 7, dtype=torch.int32, device=gu.dev())
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_layer_forward_static(cfg, sentinel, sentinel, sentinel, sentinel, None, None,
                                     sentinel, sentinel, sentinel, sentinel, sentinel)
    assert ei.value.status == -3   # MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (sentinel.cpu() == 7).all()
