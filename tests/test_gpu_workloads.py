"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark times (moe_layer_forward on the whole batch).

Routing ids, expert counts, balancedness and the whole permutation
(seg_offsets, seg_expert, assign_to_row, row_to_token) are compared with the
oracle bit for bit over the full batch.  The layer output and the grouped-FFN
rows are compared on a sample of tokens (first, last, random, tokens of the
hottest expert and of both replicas of a split expert), each computed by the
oracle from the definition out[t] = sum_j w_tj SwiGLU_e(x_t) (+ shared).
The FP8-weight variants run the same layers through moe_layer_forward_fp8w
with the library's own quantization of the drawn weights; the oracle
quantizes the same weights itself (their codes are compared bit for bit for
every expert the sample needs) and computes with the dequantized values."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import fp8 as ofp8
from oracle import moe_oracle as orc
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _sample_tokens(cfg, ids, rng):
    T = cfg.T
    n_rand = 10 if cfg.weights != "fp8" else 3     # FP8: the oracle quantizes each expert needed
    toks = {0, T - 1} | set(rng.choice(T, size=min(T, n_rand), replace=False).tolist())
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    hot = int(np.argmax(counts))
    users = np.nonzero((ids == hot).any(axis=1))[0]
    for parity in (0, 1):
        sel = users[users % 2 == parity]
        toks |= set(sel[:2].tolist())
    toks |= set(users[-2:].tolist())   # the last replica of a load-bounded split
    return np.array(sorted(toks))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_fp32", "decode_bf16", "prefill_skew_bf16",
                                  "ragged_stress_bf16", "deepseek_v3_bf16", "decode_fp8w",
                                  "prefill_skew_fp8w", "ragged_stress_fp8w", "deepseek_v3_fp8w",
                                  "ragged_stress_bounded_bf16", "decode_capacity_bf16",
                                  "decode_w8a8", "prefill_skew_w8a8", "ragged_stress_w8a8",
                                  "deepseek_v3_w8a8"])
def test_workload_full_size(name):
    import mixture_experts_layer_segments_amd as moe
    cfg = mi.WORKLOADS[name]
    print(f"\n[workload] {name}: routing on the host", flush=True)
    logits = mi.logits(cfg)
    ids_r, w_r, gap = orc.route(cfg, logits)
    plan_r = orc.plan(cfg, ids_r)
    rng = np.random.default_rng(cfg.seed)
    toks = _sample_tokens(cfg, ids_r, rng)
    xb = mi.x(cfg)
    x64_s = mi.values_f64(xb[toks], cfg.dtype)
    need = {}
    for i, t in enumerate(toks):
        for j, e in enumerate(ids_r[t].tolist()):
            need.setdefault(e, []).append((i, j))

    dev = gu.dev()
    tdt = gu.tdtype(cfg)
    w13_d = torch.empty((cfg.E, 2 * cfg.I, cfg.H), dtype=tdt, device=dev)
    w2_d = torch.empty((cfg.E, cfg.H, cfg.I), dtype=tdt, device=dev)
    y_ref = {}   # (i, j) -> oracle expert output row (unweighted)
    slack_ref = {}   # W8A8: (i, j) -> h-code slack of that row (unweighted)
    codes_ref = {}   # FP8: expert -> oracle codes and scales of (w13, w2)

    def weights64(a, b):
        a64, b64 = mi.values_f64(a, cfg.dtype), mi.values_f64(b, cfg.dtype)
        if cfg.weights != "fp8":
            return a64, b64, None
        qa, qb = ofp8.quantize_blocks(a64), ofp8.quantize_blocks(b64)
        return ofp8.dequantize_blocks(*qa), ofp8.dequantize_blocks(*qb), (qa, qb)

    def expert(x_rows, a64, b64):
        if cfg.acts == "fp8":      # x quantized in 1 x 128 pieces, h too (W8A8)
            return ofp8.expert_w8a8(ofp8.fake_quant_rows(x_rows), a64, b64)
        return orc.swiglu(x_rows, a64, b64)

    def put(e, a, b):
        w13_d[e].copy_(gu.to_dev(a, cfg.dtype))
        w2_d[e].copy_(gu.to_dev(b, cfg.dtype))
        if e in need:
            rows = [i for i, _ in need[e]]
            a64, b64, q = weights64(a, b)
            if q is not None:
                codes_ref[e] = q
            y = expert(x64_s[rows], a64, b64)
            sl = (gu.h_code_slack(ofp8.fake_quant_rows(x64_s[rows]), a64, b64)
                  if cfg.acts == "fp8" else np.zeros_like(y))
            for n, (i, j) in enumerate(need[e]):
                y_ref[(i, j)] = y[n]
                slack_ref[(i, j)] = sl[n]

    print(f"[workload] {name}: generating {cfg.E} experts", flush=True)
    mi.for_each_expert(cfg, put)
    out_ref = np.zeros((len(toks), cfg.H))
    out_slack = np.zeros((len(toks), cfg.H))
    kept = plan_r["assign_to_row"] >= 0          # the fixed-capacity layout drops some
    for (i, j), y in y_ref.items():
        if kept[toks[i] * cfg.k + j]:
            out_ref[i] += w_r[toks[i], j] * y
            out_slack[i] += w_r[toks[i], j] * slack_ref[(i, j)]
    d = dict(logits=torch.from_numpy(logits).to(dev), x=gu.to_dev(xb, cfg.dtype), w13=w13_d,
             w2=w2_d, sw13=None, sw2=None)
    if cfg.shared_I:
        s13, s2 = mi.shared_w13(cfg), mi.shared_w2(cfg)
        a64, b64, _ = weights64(s13, s2)
        out_ref += expert(x64_s, a64, b64)
        if cfg.acts == "fp8":
            out_slack += gu.h_code_slack(ofp8.fake_quant_rows(x64_s), a64, b64)
        d["sw13"], d["sw2"] = gu.to_dev(s13, cfg.dtype), gu.to_dev(s2, cfg.dtype)
    torch.cuda.synchronize()

    print(f"[workload] {name}: layer forward", flush=True)
    o = gu.run_layer(moe, cfg, d)
    if cfg.weights == "fp8":
        q = o["q"]
        for e, (qa, qb) in codes_ref.items():
            assert np.array_equal(q["w13"][e].cpu().numpy(), qa[0]), f"w13 codes of expert {e}"
            assert np.array_equal(q["w13_s"][e].cpu().numpy().astype(np.float64), qa[1]), e
            assert np.array_equal(q["w2"][e].cpu().numpy(), qb[0]), f"w2 codes of expert {e}"
            assert np.array_equal(q["w2_s"][e].cpu().numpy().astype(np.float64), qb[1]), e
        print(f"[workload] {name}: codes of {len(codes_ref)} experts match", flush=True)
    ids_g = o["ids"].cpu().numpy()
    mism = gu.check_routing(cfg, ids_g, o["w"].cpu().numpy(), ids_r, w_r, gap, logits)
    if mism.size == 0:
        gu.check_plan(o, plan_r)      # the permutation the layer built, bit for bit
    assert (o["counts"].cpu().numpy() == plan_r["counts"]).all()
    assert o["bal"].cpu().numpy()[0] == plan_r["balancedness"]
    got = gu.host_f64(o["out"][torch.from_numpy(toks).to(dev)])
    ok = ~np.isin(toks, mism)
    err = gu.rel_err(got[ok], out_ref[ok])
    print(f"[workload] {name}: sampled {ok.sum()} tokens, rel err {err:.3e}, "
          f"balancedness {o['bal'].item():.4f}", flush=True)
    if cfg.acts == "fp8":
        gu.check_w8a8_out(got[ok], out_ref[ok], out_slack[ok], name + " layer")
    else:
        assert err <= gu.rel_tol(cfg), err

    if mism.size == 0:
        print(f"[workload] {name}: permutation + grouped FFN steps", flush=True)
        g = gu.run_permute(moe, cfg, d["x"], o["ids"])
        gu.check_plan(g, plan_r)
        a2r = plan_r["assign_to_row"]
        pairs = [(i, j) for i, t in enumerate(toks) for j in range(cfg.k) if kept[t * cfg.k + j]]
        rows = torch.from_numpy(np.array([a2r[toks[i] * cfg.k + j] for i, j in pairs])).long().to(dev)
        tok_rows = torch.from_numpy(np.array([toks[i] for i, _ in pairs])).long().to(dev)
        xv = g["x_perm"][rows].cpu()
        xs = d["x"][tok_rows].cpu()
        assert torch.equal(xv.view(torch.int16) if cfg.dtype == "bf16" else xv,
                           xs.view(torch.int16) if cfg.dtype == "bf16" else xs)
        y = torch.empty_like(g["x_perm"])
        ws = gu.empty((moe.moe_workspace_size(cfg),), torch.uint8)
        if cfg.acts == "fp8":
            q = o["q"]
            xq, xs = gu.quantize_act(moe, g["x_perm"])
            moe.moe_grouped_ffn_w8a8(cfg, xq, xs, g["seg_offsets"], g["seg_expert"], q["w13"],
                                     q["w13_s"], q["w2"], q["w2_s"], None, y, ws)
        elif cfg.weights == "fp8":
            q = o["q"]
            moe.moe_grouped_ffn_fp8w(cfg, g["x_perm"], g["seg_offsets"], g["seg_expert"],
                                     q["w13"], q["w13_s"], q["w2"], q["w2_s"], None, y, ws)
        else:
            moe.moe_grouped_ffn(cfg, g["x_perm"], g["seg_offsets"], g["seg_expert"], w13_d,
                                w2_d, None, y, ws)
        torch.cuda.synchronize()
        yg = gu.host_f64(y[rows])
        yr = np.stack([y_ref[p] for p in pairs])
        err = gu.rel_err(yg, yr)
        print(f"[workload] {name}: grouped FFN sampled rows rel err {err:.3e}", flush=True)
        if cfg.acts == "fp8":
            gu.check_w8a8_out(yg, yr, np.stack([slack_ref[p] for p in pairs]), name + " FFN")
        else:
            assert err <= gu.rel_tol(cfg), err
