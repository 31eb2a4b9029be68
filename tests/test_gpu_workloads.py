"""GPU parity at the full sizes of the workloads, in the launch configuration
the benchmark times (moe_layer_forward on the whole batch).

For every workload:
* routing ids, expert counts, balancedness and the layer's whole permutation
  (seg_offsets, seg_expert, assign_to_row, row_to_token) bit for bit over the
  whole batch.  Where a DeepSeek-shaped token's kept groups sit within a few
  fp32 ulp of a tie, either choice is correct (check_routing shows the GPU's
  is valid); the oracle then rebuilds the plan from the GPU's ids and that is
  compared bit for bit, and the token's expected output uses those ids;
* moe_permute on the GPU's ids: the same permutation bit for bit, and x_perm
  byte for byte on the rows compared below.

bf16 and fp32 layers ("Follow one token through an MoE layer", steps 3-4):
* the whole layer output, every element of every token, against the
  oracle's out[t] = sum_j w_tj SwiGLU_e(x_t) (+ the shared expert), computed
  from that definition expert by expert over all of the expert's tokens;
* moe_grouped_ffn on moe_permute's rows: every live row of y_perm on the
  decode and prefill layers; on the larger ones the first and last row of
  every segment and one row inside every 256-row tile.

FP8 layers (moe_layer_forward_fp8w / _w8a8 with the library's own
quantization of the drawn weights; the oracle quantizes the same weights
itself): the oracle's block quantizer takes seconds per expert, so these
compare a sample -- the layer output of sampled tokens (first, last, random,
users of the hottest expert and of its replicas), and y_perm rows of the
two hottest experts and three others (first and last row of every segment
of theirs and one row in every 256-row tile), with the weight codes of every
expert the sample needs compared bit for bit.
"""
import time

import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import fp8 as ofp8
from oracle import moe_oracle as orc
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

WHOLE = ["tiny_fp32", "decode_bf16", "prefill_skew_bf16", "ragged_stress_bf16",
         "deepseek_v3_bf16", "ragged_stress_bounded_bf16", "decode_capacity_bf16"]
FP8 = ["decode_fp8w", "prefill_skew_fp8w", "ragged_stress_fp8w", "deepseek_v3_fp8w",
       "decode_w8a8", "prefill_skew_w8a8", "ragged_stress_w8a8", "deepseek_v3_w8a8"]
EVERY_ROW = {"tiny_fp32", "decode_bf16", "prefill_skew_bf16", "decode_capacity_bf16"}

# Whole-layer oracle outputs, shared by workloads with the same inputs and
# routing: a replica split moves rows between segments, not results.
_OUT_CACHE = {}


def _say(name, t0, msg):
    print(f"[workload] {name} +{time.perf_counter() - t0:.1f}s: {msg}", flush=True)


def _routing_used(cfg, logits, ids_r, w_r, gap, ids_g, w_g):
    """The oracle's ids and weights, with any token whose group choice sits on
    a tie taken as the GPU chose it (check_routing has shown it is valid)."""
    mism = gu.check_routing(cfg, ids_g, w_g, ids_r, w_r, gap, logits)
    if mism.size == 0:
        return ids_r, w_r, mism
    ids_u, w_u = ids_r.copy(), w_r.copy()
    ids_u[mism] = ids_g[mism]
    w_u[mism] = orc.sigmoid_weights(logits[mism], ids_g[mism], bool(cfg.renormalize))
    return ids_u, w_u, mism


def _check_x_perm(cfg, g, d, plan, rows):
    tok = torch.from_numpy(plan["row_to_token"][rows].astype(np.int64)).to(gu.dev())
    rr = torch.from_numpy(rows).to(gu.dev())
    xv, xs = g["x_perm"][rr].cpu(), d["x"][tok].cpu()
    view = (lambda t: t.view(torch.int16)) if cfg.dtype == "bf16" else (lambda t: t)
    assert torch.equal(view(xv), view(xs)), "x_perm rows differ from their tokens' rows"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", WHOLE)
def test_workload_whole_output(name):
    import mixture_experts_layer_segments_amd as moe
    cfg = mi.WORKLOADS[name]
    t0 = time.perf_counter()
    _say(name, t0, "routing on the host")
    logits = mi.logits(cfg)
    ids_r, w_r, gap = orc.route(cfg, logits)
    xb = mi.x(cfg)
    x64 = mi.values_f64(xb, cfg.dtype)
    dev, tdt = gu.dev(), gu.tdtype(cfg)
    w13_d = torch.empty((cfg.E, 2 * cfg.I, cfg.H), dtype=tdt, device=dev)
    w2_d = torch.empty((cfg.E, cfg.H, cfg.I), dtype=tdt, device=dev)

    def upload(e, a, b):
        w13_d[e].copy_(gu.to_dev(a, cfg.dtype))
        w2_d[e].copy_(gu.to_dev(b, cfg.dtype))

    d = dict(logits=torch.from_numpy(logits).to(dev), x=gu.to_dev(xb, cfg.dtype), w13=w13_d,
             w2=w2_d, sw13=None, sw2=None)
    if cfg.shared_I:
        d["sw13"] = gu.to_dev(mi.shared_w13(cfg), cfg.dtype)
        d["sw2"] = gu.to_dev(mi.shared_w2(cfg), cfg.dtype)
    _say(name, t0, f"drawing {cfg.E} experts onto the device")
    mi.for_each_expert(cfg, upload)
    torch.cuda.synchronize()

    _say(name, t0, "layer forward on the GPU")
    o = gu.run_layer(moe, cfg, d)
    ids_u, w_u, mism = _routing_used(cfg, logits, ids_r, w_r, gap, o["ids"].cpu().numpy(),
                                     o["w"].cpu().numpy())
    if mism.size:
        _say(name, t0, f"{mism.size} tokens on a group tie: plan rebuilt from the GPU's ids")
    plan = orc.plan(cfg, ids_u)
    gu.check_plan(o, plan)
    assert (o["counts"].cpu().numpy() == plan["counts"]).all()

    _say(name, t0, "permutation and grouped FFN on the GPU")
    g = gu.run_permute(moe, cfg, d["x"], o["ids"])
    gu.check_plan(g, plan)
    R = int(plan["seg_offsets"][-1])
    if name in EVERY_ROW:
        rows = np.nonzero(plan["row_to_token"][:R] >= 0)[0].astype(np.int64)
    else:
        rows = gu.segment_sample_rows(plan, np.random.default_rng(cfg.seed))
    _check_x_perm(cfg, g, d, plan, rows)
    y = torch.empty_like(g["x_perm"])
    ws = gu.empty((moe.moe_workspace_size(cfg),), torch.uint8)
    moe.moe_grouped_ffn(cfg, g["x_perm"], g["seg_offsets"], g["seg_expert"], w13_d, w2_d, None,
                        y, ws)
    torch.cuda.synchronize()
    y_got = gu.host_f64(y[torch.from_numpy(rows).to(dev)])
    out_got = gu.host_f64(o["out"])
    del w13_d, w2_d, y, ws, g
    torch.cuda.empty_cache()

    # the oracle, expert by expert over every token that routes to it
    k = cfg.k
    want_a = np.sort(plan["row_to_assign"][rows].astype(np.int64))   # assignments of the rows
    kept = plan["assign_to_row"] >= 0
    key = (cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.shared_I, cfg.seed, cfg.dtype, cfg.score,
           cfg.capacity_factor_permille)
    y_want = np.zeros((want_a.size, cfg.H))
    out_ref = _OUT_CACHE.get(key) if mism.size == 0 else None
    acc = np.zeros((cfg.T, cfg.H)) if out_ref is None else None

    def oracle_expert(e, a, b):
        sel = np.nonzero((ids_u.ravel() == e) & kept)[0]
        hit = np.isin(sel, want_a)
        todo = sel if acc is not None else sel[hit]    # (only the wanted rows when cached)
        if todo.size == 0:
            return
        a64, b64 = mi.values_f64(a, cfg.dtype), mi.values_f64(b, cfg.dtype)
        t = todo // k
        ye = orc.swiglu(x64[t], a64, b64)
        if acc is not None:
            assert np.unique(t).size == t.size        # distinct experts per token
            acc[t] += w_u.ravel()[todo][:, None] * ye
            y_want[np.searchsorted(want_a, todo[hit])] = ye[hit]
        else:
            y_want[np.searchsorted(want_a, todo)] = ye

    _say(name, t0, "oracle over every expert's tokens" if acc is not None else
         "oracle over the compared rows (layer output cached from the same routing)")
    mi.for_each_expert(cfg, oracle_expert)
    if acc is not None:
        if cfg.shared_I:
            acc += orc.swiglu(x64, mi.values_f64(mi.shared_w13(cfg), cfg.dtype),
                              mi.values_f64(mi.shared_w2(cfg), cfg.dtype))
        out_ref = acc
        if mism.size == 0:
            _OUT_CACHE.clear()
            _OUT_CACHE[key] = out_ref

    err = gu.rel_err(out_got, out_ref)
    _say(name, t0, f"whole output, {cfg.T} x {cfg.H}: rel err {err:.3e} "
         f"(balancedness {o['bal'].item():.4f})")
    assert err <= gu.rel_tol(cfg), err
    # y_perm rows, in the order of `rows`: map each wanted assignment back
    pos = np.searchsorted(want_a, plan["row_to_assign"][rows].astype(np.int64))
    err_y = gu.rel_err(y_got, y_want[pos])
    _say(name, t0, f"grouped FFN, {rows.size} of {R} rows: rel err {err_y:.3e}")
    assert err_y <= gu.rel_tol(cfg), err_y


def _sample_tokens(cfg, ids, rng):
    T = cfg.T
    toks = {0, T - 1} | set(rng.choice(T, size=min(T, 3), replace=False).tolist())
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    hot = int(np.argmax(counts))
    users = np.nonzero((ids == hot).any(axis=1))[0]
    for parity in (0, 1):
        sel = users[users % 2 == parity]
        toks |= set(sel[:2].tolist())
    toks |= set(users[-2:].tolist())   # the last replica of a load-bounded split
    return np.array(sorted(toks))


def _fp8_row_experts(plan, rng, n_other=3):
    """The two experts with the most rows and n_other other active ones."""
    counts = plan["counts"]
    order = np.argsort(-counts, kind="stable")
    hot = [int(e) for e in order[:2] if counts[e] > 0]
    rest = [int(e) for e in np.nonzero(counts > 0)[0] if int(e) not in hot]
    other = rng.choice(rest, size=min(n_other, len(rest)), replace=False).tolist() if rest else []
    return hot + [int(e) for e in other]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FP8)
def test_workload_fp8_sampled(name):
    import mixture_experts_layer_segments_amd as moe
    cfg = mi.WORKLOADS[name]
    t0 = time.perf_counter()
    _say(name, t0, "routing on the host")
    logits = mi.logits(cfg)
    ids_r, w_r, gap = orc.route(cfg, logits)
    plan_r = orc.plan(cfg, ids_r)
    rng = np.random.default_rng(cfg.seed)
    toks = _sample_tokens(cfg, ids_r, rng)
    xb = mi.x(cfg)
    x64 = mi.values_f64(xb, cfg.dtype)
    xq64 = ofp8.fake_quant_rows(x64) if cfg.acts == "fp8" else x64
    # y_perm rows of a few experts: first / last row of each of their
    # segments and one row in every 256-row tile
    row_experts = _fp8_row_experts(plan_r, rng)
    seg_rows = gu.segment_sample_rows(plan_r, rng)
    seg_of = np.searchsorted(plan_r["seg_offsets"], seg_rows, side="right") - 1
    rows = seg_rows[np.isin(plan_r["seg_expert"][seg_of], row_experts)]
    row_a = plan_r["row_to_assign"][rows].astype(np.int64)
    need = {}
    for i, t in enumerate(toks):
        for j, e in enumerate(ids_r[t].tolist()):
            need.setdefault(e, set()).add(int(t))
    for a in row_a:
        need.setdefault(int(ids_r.ravel()[a]), set()).add(int(a // cfg.k))

    dev, tdt = gu.dev(), gu.tdtype(cfg)
    w13_d = torch.empty((cfg.E, 2 * cfg.I, cfg.H), dtype=tdt, device=dev)
    w2_d = torch.empty((cfg.E, cfg.H, cfg.I), dtype=tdt, device=dev)
    y_tok = {}       # (token, expert) -> oracle expert output (unweighted)
    slack_tok = {}   # W8A8: (token, expert) -> h-code slack of that row
    codes_ref = {}   # expert -> oracle codes and scales of (w13, w2)

    def expert(x_rows, a64, b64):
        if cfg.acts == "fp8":
            return ofp8.expert_w8a8(x_rows, a64, b64)
        return orc.swiglu(x_rows, a64, b64)

    def put(e, a, b):
        w13_d[e].copy_(gu.to_dev(a, cfg.dtype))
        w2_d[e].copy_(gu.to_dev(b, cfg.dtype))
        if e not in need:
            return
        qa = gu.quantize_blocks_strips(mi.values_f64(a, cfg.dtype))
        qb = gu.quantize_blocks_strips(mi.values_f64(b, cfg.dtype))
        codes_ref[e] = (qa, qb)
        a64, b64 = ofp8.dequantize_blocks(*qa), ofp8.dequantize_blocks(*qb)
        tl = np.array(sorted(need[e]))
        y = expert(xq64[tl], a64, b64)
        sl = (gu.h_code_slack(xq64[tl], a64, b64) if cfg.acts == "fp8" else np.zeros_like(y))
        for n, t in enumerate(tl.tolist()):
            y_tok[(t, e)] = y[n]
            slack_tok[(t, e)] = sl[n]

    _say(name, t0, f"drawing {cfg.E} experts; the oracle quantizes the {len(need)} it needs")
    mi.for_each_expert(cfg, put)
    d = dict(logits=torch.from_numpy(logits).to(dev), x=gu.to_dev(xb, cfg.dtype), w13=w13_d,
             w2=w2_d, sw13=None, sw2=None)
    shared_ref = shared_slack = None
    if cfg.shared_I:
        s13, s2 = mi.shared_w13(cfg), mi.shared_w2(cfg)
        a64 = ofp8.dequantize_blocks(*gu.quantize_blocks_strips(mi.values_f64(s13, cfg.dtype)))
        b64 = ofp8.dequantize_blocks(*gu.quantize_blocks_strips(mi.values_f64(s2, cfg.dtype)))
        shared_ref = expert(xq64[toks], a64, b64)
        if cfg.acts == "fp8":
            shared_slack = gu.h_code_slack(xq64[toks], a64, b64)
        d["sw13"], d["sw2"] = gu.to_dev(s13, cfg.dtype), gu.to_dev(s2, cfg.dtype)
    torch.cuda.synchronize()

    _say(name, t0, "layer forward on the GPU")
    o = gu.run_layer(moe, cfg, d)
    q = o["q"]
    for e, (qa, qb) in codes_ref.items():
        assert np.array_equal(q["w13"][e].cpu().numpy(), qa[0]), f"w13 codes of expert {e}"
        assert np.array_equal(q["w13_s"][e].cpu().numpy().astype(np.float64), qa[1]), e
        assert np.array_equal(q["w2"][e].cpu().numpy(), qb[0]), f"w2 codes of expert {e}"
        assert np.array_equal(q["w2_s"][e].cpu().numpy().astype(np.float64), qb[1]), e
    _say(name, t0, f"weight codes of {len(codes_ref)} experts match")
    ids_g = o["ids"].cpu().numpy()
    ids_u, w_u, mism = _routing_used(cfg, logits, ids_r, w_r, gap, ids_g, o["w"].cpu().numpy())
    plan = orc.plan(cfg, ids_u) if mism.size else plan_r
    gu.check_plan(o, plan)
    assert (o["counts"].cpu().numpy() == plan["counts"]).all()

    # layer output of the sampled tokens whose experts the oracle computed
    ok = np.array([all((int(t), int(e)) in y_tok for e in ids_u[t]) for t in toks])
    tk = toks[ok]
    out_ref = np.zeros((tk.size, cfg.H))
    out_slack = np.zeros((tk.size, cfg.H))
    kept = plan["assign_to_row"] >= 0
    for i, t in enumerate(tk.tolist()):
        for j, e in enumerate(ids_u[t].tolist()):
            if kept[t * cfg.k + j]:
                out_ref[i] += w_u[t, j] * y_tok[(t, e)]
                out_slack[i] += w_u[t, j] * slack_tok[(t, e)]
    if shared_ref is not None:
        out_ref += shared_ref[ok]
        if shared_slack is not None:
            out_slack += shared_slack[ok]
    got = gu.host_f64(o["out"][torch.from_numpy(tk).to(dev)])
    _say(name, t0, f"layer output of {tk.size} sampled tokens: rel err {gu.rel_err(got, out_ref):.3e}")
    if cfg.acts == "fp8":
        gu.check_w8a8_out(got, out_ref, out_slack, name + " layer")
    else:
        assert gu.rel_err(got, out_ref) <= gu.rel_tol(cfg)

    # grouped FFN on moe_permute's rows: the sampled tokens' rows and the
    # segment rows of the chosen experts
    g = gu.run_permute(moe, cfg, d["x"], o["ids"])
    gu.check_plan(g, plan)
    a2r = plan["assign_to_row"]
    pairs = [(int(t), j) for t in tk for j in range(cfg.k) if kept[t * cfg.k + j]]
    pairs += [(int(a // cfg.k), int(a % cfg.k)) for a in row_a if int(a // cfg.k) not in mism]
    pairs = sorted(set(pairs))
    cmp_rows = np.array([a2r[t * cfg.k + j] for t, j in pairs], dtype=np.int64)
    _check_x_perm(cfg, g, d, plan, cmp_rows)
    y = torch.empty_like(g["x_perm"])
    ws = gu.empty((moe.moe_workspace_size(cfg),), torch.uint8)
    if cfg.acts == "fp8":
        xq, xs = gu.quantize_act(moe, g["x_perm"])
        moe.moe_grouped_ffn_w8a8(cfg, xq, xs, g["seg_offsets"], g["seg_expert"], q["w13"],
                                 q["w13_s"], q["w2"], q["w2_s"], None, y, ws)
    else:
        moe.moe_grouped_ffn_fp8w(cfg, g["x_perm"], g["seg_offsets"], g["seg_expert"], q["w13"],
                                 q["w13_s"], q["w2"], q["w2_s"], None, y, ws)
    torch.cuda.synchronize()
    yg = gu.host_f64(y[torch.from_numpy(cmp_rows).to(dev)])
    yr = np.stack([y_tok[(t, int(ids_u[t, j]))] for t, j in pairs])
    _say(name, t0, f"grouped FFN, {len(pairs)} rows ({rows.size} from the segments of experts "
         f"{row_experts}): rel err {gu.rel_err(yg, yr):.3e}")
    if cfg.acts == "fp8":
        ys = np.stack([slack_tok[(t, int(ids_u[t, j]))] for t, j in pairs])
        gu.check_w8a8_out(yg, yr, ys, name + " FFN")
    else:
        assert gu.rel_err(yg, yr) <= gu.rel_tol(cfg)
