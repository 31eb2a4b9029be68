"""The library is re-entrant across streams when the workspaces differ: two
host threads, each with its own stream, workspace and outputs, run
moe_layer_forward on different batches at the same time (the first calls of
each kernel shape included, so the launch-configuration caches are filled
concurrently), and every result equals, bit for bit, the same call made
alone."""
import threading

import numpy as np
import pytest
import torch

import moe_inputs as mi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _layer(moe, cfg, d, stream):
    tdt = gu.tdtype(cfg)
    with torch.cuda.stream(stream):
        o = dict(out=gu.empty((cfg.T, cfg.H), tdt), ids=gu.empty((cfg.T, cfg.k), torch.int32),
                 w=gu.empty((cfg.T, cfg.k), torch.float32), counts=gu.empty((cfg.E,), torch.int32),
                 bal=gu.empty((1,), torch.float32))
        ws = gu.empty((moe.moe_workspace_size(cfg),), torch.uint8)
        moe.moe_layer_forward(cfg, d["logits"], d["x"], d["w13"], d["w2"], d["sw13"], d["sw2"],
                              o["out"], o["ids"], o["w"], o["counts"], o["bal"], ws)
    stream.synchronize()
    return o


def test_two_threads_two_streams():
    import mixture_experts_layer_segments_amd as moe
    cfgs = [mi.MoEShape("s1", T=300, H=512, E=16, k=4, I=256, zipf_s=1.2, seed=61),
            mi.MoEShape("s2", T=1100, H=384, E=3, k=1, I=256, zipf_s=1.0, seed=62)]
    cases = [gu.SmallCase(c) for c in cfgs]
    inputs = [c.device_inputs() for c in cases]
    torch.cuda.synchronize()
    got = [None, None]
    errors = []

    def run(i):
        try:
            s = torch.cuda.Stream()
            for _ in range(3):
                got[i] = _layer(moe, cfgs[i], inputs[i], s)
        except Exception as e:   # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(2):
        alone = _layer(moe, cfgs[i], inputs[i], torch.cuda.current_stream())
        for key in alone:
            a, b = alone[key], got[i][key]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (cfgs[i].name, key)
        err = gu.rel_err(gu.host_f64(got[i]["out"]), cases[i].ref["out"])
        assert err <= gu.BF16_REL, err
        assert np.array_equal(got[i]["ids"].cpu().numpy(), cases[i].ref["ids"])
