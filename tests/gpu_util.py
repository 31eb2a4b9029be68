"""Helpers shared by the GPU parity tests: seeded inputs on the device, the
C-ABI calls, and the oracle's expected values (computed on the host from the
same seeded inputs; nothing expected ever comes from the GPU)."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs as mi
from oracle import fp8 as ofp8
from oracle import moe_oracle as orc

BF16_REL = 1.5e-2   # max|gpu - oracle| <= BF16_REL * max|oracle|  (bf16 layers)
F32_REL = 1e-4      # same, fp32 layers
W_TOL = 2.0 ** -24  # routing weights: fp64 math rounded once to fp32


def dev():
    return torch.device("cuda:0")


def tdtype(cfg):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def to_dev(a: np.ndarray, dtype: str):
    """Host input (fp32 array or bf16 bits) -> device tensor of that type."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))


def rel_tol(cfg) -> float:
    return F32_REL if cfg.dtype == "f32" else BF16_REL


def empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device=dev())


class SmallCase:
    """A layer small enough for the whole oracle: all inputs on host and
    device, and every intermediate of the oracle."""

    def __init__(self, cfg, logits=None, ids_override=None):
        self.cfg = cfg
        self.logits = mi.logits(cfg) if logits is None else logits
        self.xb = mi.x(cfg)
        self.w13b = np.stack([mi.w13(cfg, e) for e in range(cfg.E)])
        self.w2b = np.stack([mi.w2(cfg, e) for e in range(cfg.E)])
        self.sw13b = mi.shared_w13(cfg) if cfg.shared_I else None
        self.sw2b = mi.shared_w2(cfg) if cfg.shared_I else None
        f = lambda a: None if a is None else mi.values_f64(a, cfg.dtype)  # noqa: E731
        self.x64, self.w13_64, self.w2_64 = f(self.xb), f(self.w13b), f(self.w2b)
        self.sw13_64, self.sw2_64 = f(self.sw13b), f(self.sw2b)
        if cfg.weights == "fp8":
            # the oracle quantizes the same drawn weights itself and runs the
            # layer on the dequantized values
            self.q = {}
            for name in ("w13", "w2", "sw13", "sw2"):
                w = getattr(self, name + "_64")
                if w is None:
                    continue
                mats = w if w.ndim == 3 else w[None]
                qs = [ofp8.quantize_blocks(m) for m in mats]
                codes = np.stack([c for c, _ in qs])
                scales = np.stack([sc for _, sc in qs])
                self.q[name] = (codes, scales)
                deq = np.stack([ofp8.dequantize_blocks(c, sc) for c, sc in qs])
                setattr(self, name + "_64", deq if w.ndim == 3 else deq[0])
        if cfg.acts == "fp8":
            self.ref = ofp8.layer_forward_w8a8(cfg, self.logits, self.x64, self.w13_64,
                                               self.w2_64, self.sw13_64, self.sw2_64)
        else:
            self.ref = orc.layer_forward(cfg, self.logits, self.x64, self.w13_64, self.w2_64,
                                         self.sw13_64, self.sw2_64)

    def device_inputs(self):
        c = self.cfg
        d = dict(logits=torch.from_numpy(self.logits).to(dev()), x=to_dev(self.xb, c.dtype),
                 w13=to_dev(self.w13b, c.dtype), w2=to_dev(self.w2b, c.dtype),
                 sw13=None, sw2=None)
        if c.shared_I:
            d["sw13"] = to_dev(self.sw13b, c.dtype)
            d["sw2"] = to_dev(self.sw2b, c.dtype)
        return d


def h_code_slack(xq_rows, w13_e, w2_e) -> np.ndarray:
    """W8A8: how far an expert's output rows [n, H] may move because the GPU
    decides h's E4M3 codes on its own fp32 sums.  The GPU's h may differ from
    the oracle's float64 h by about the rounding of a K-term fp32 sum; the
    band used is 2^-20 sqrt(K) times the root-sum-square of the terms, 16 x
    the usual size of that error, plus 2^-20 |h|.  Where the band around an
    element holds two codes (after the bf16 rounding, at the oracle's piece
    scale), or the band around a piece's maximum holds two scales, that
    element's dequantized h may differ by one E4M3 step; the slack of an
    output element is the sum of those steps times |W2|."""
    I = w13_e.shape[0] // 2
    K = xq_rows.shape[1]
    wg, wu = w13_e[:I], w13_e[I:]
    g, u = xq_rows @ wg.T, xq_rows @ wu.T
    g2 = np.sqrt((xq_rows ** 2) @ (wg ** 2).T)
    u2 = np.sqrt((xq_rows ** 2) @ (wu ** 2).T)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = np.abs(sig * (1.0 + g * (1.0 - sig)))
    h = silu * u
    dh = 2.0 ** -20 * np.sqrt(K) * (dsilu * np.abs(u) * g2 + np.abs(silu) * u2) + \
        2.0 ** -20 * np.abs(h)
    hb = ofp8.bf16_round(h)
    n = h.shape[0]
    _, sc = ofp8.quantize_rows(hb)
    s_rep = np.repeat(sc, 128, axis=1)
    two_codes = (ofp8.e4m3_encode(ofp8.bf16_round(h - dh) / s_rep) !=
                 ofp8.e4m3_encode(ofp8.bf16_round(h + dh) / s_rep))
    amax_lo = np.maximum(np.abs(h) - dh, 0.0).reshape(n, -1, 128).max(axis=2)
    amax_hi = (np.abs(h) + dh).reshape(n, -1, 128).max(axis=2)
    s_lo = ofp8.scale_exponents(ofp8.bf16_round(amax_lo))
    s_hi = ofp8.scale_exponents(ofp8.bf16_round(amax_hi))
    two_scales = np.repeat(s_lo != s_hi, 128, axis=1)
    step = 2.0 ** -3 * np.abs(hb) + 2.0 ** -9 * np.repeat(2.0 ** s_hi, 128, axis=1)
    return np.where(two_codes | two_scales, step, 0.0) @ np.abs(w2_e).T


def w8a8_slack(case) -> np.ndarray:
    """h_code_slack of every token of a SmallCase, summed over its routed
    slots with their router weights (and the shared expert)."""
    c, r = case.cfg, case.ref
    xq = ofp8.fake_quant_rows(case.x64)
    out = np.zeros((c.T, c.H))
    kept = r["assign_to_row"].reshape(c.T, c.k) >= 0
    for e in range(c.E):
        t, j = np.nonzero((r["ids"] == e) & kept)
        if t.size:
            out[t] += r["w"][t, j][:, None] * h_code_slack(xq[t], case.w13_64[e], case.w2_64[e])
    if c.shared_I:
        out += h_code_slack(xq, case.sw13_64, case.sw2_64)
    return out


# At most this fraction of the output elements may carry an h-code slack
# larger than the plain tolerance itself (measured on the small W8A8 layers:
# 0 to 0.41%); a looser slack would stop the check from meaning anything.
W8A8_BIG_SLACK_FRAC = 0.01


def check_w8a8_out(got, ref, slack, name=""):
    """|got - ref| within the bf16 layer tolerance plus the per-element
    h-code slack; returns the largest error beyond the slack, relative.
    Fails too when more than W8A8_BIG_SLACK_FRAC of the elements carry a
    slack above the plain tolerance."""
    m = np.abs(ref).max()
    excess = (np.abs(got - ref) - slack) / m
    worst = float(excess.max())
    flagged = int((slack > 0).any(axis=1).sum())
    big = float(np.mean(slack > BF16_REL * m))
    print(f"  {name}: error beyond the h-code slack {worst:.3e} (raw "
          f"{np.abs(got - ref).max() / m:.3e}; {flagged} of {len(ref)} rows with slack, "
          f"{100 * big:.3f}% of elements with slack above the tolerance)", flush=True)
    assert big <= W8A8_BIG_SLACK_FRAC, big
    assert worst <= BF16_REL, worst
    return worst


def quantize_blocks_strips(w64, threads=None):
    """The oracle's quantize_blocks on a matrix, one strip of 128 rows at a
    time in a thread pool (numpy releases the GIL in its kernels).  Every
    128 x 128 block is quantized on its own, so this is the same result as
    one call on the whole matrix (a CPU test checks that), only faster."""
    from concurrent.futures import ThreadPoolExecutor
    R = w64.shape[0]
    strips = [w64[i:i + 128] for i in range(0, R, 128)]
    with ThreadPoolExecutor(max_workers=threads or mi.default_threads()) as pool:
        parts = list(pool.map(ofp8.quantize_blocks, strips))
    return (np.concatenate([c for c, _ in parts]), np.concatenate([s for _, s in parts]))


def segment_sample_rows(plan, rng, tile=256):
    """Rows of y_perm to compare when not all of them are: the first and last
    row of every computed segment, and one random row inside every 256-row
    tile of it (the big tiles' row blocks)."""
    so, se = plan["seg_offsets"], plan["seg_expert"]
    rows = set()
    for s in range(len(se)):
        r0, r1 = int(so[s]), int(so[s + 1])
        if r1 <= r0 or se[s] < 0:
            continue
        rows.update((r0, r1 - 1))
        for t0 in range(r0, r1, tile):
            rows.add(int(rng.integers(t0, min(t0 + tile, r1))))
    return np.array(sorted(rows), dtype=np.int64)


def quantize_act(moe, x):
    """The library's activation quantizer on a device bf16 tensor [R, C]:
    (codes uint8 [R, C], scales fp32 [R, C / 128])."""
    q = torch.empty(x.shape, dtype=torch.uint8, device=dev())
    sc = torch.empty((x.shape[0], x.shape[1] // 128), dtype=torch.float32, device=dev())
    moe.moe_quantize_act_fp8(x, q, sc)
    return q, sc


def x_perm_of(case):
    """The oracle's permuted rows on the device ([R, H]; padding rows of the
    fixed-capacity layout hold token 0, which no kernel reads) and the mask of
    live rows among the first seg_offsets[S]."""
    r = case.ref
    r2t = r["row_to_token"]
    R = int(r["seg_offsets"][-1])
    return to_dev(case.xb[np.maximum(r2t, 0)], case.cfg.dtype), r2t[:R] >= 0


def row_weights(case):
    """Router weight of every row (0 on padding rows), fp32."""
    r = case.ref
    r2a = r["row_to_assign"]
    w = r["w"].reshape(-1)[np.maximum(r2a, 0)]
    return np.where(r2a >= 0, w, 0.0).astype(np.float32)


def quantize_fp8(moe, w):
    """The library's block quantizer on a device bf16 tensor [.., R, C]:
    (codes uint8, scales fp32)."""
    if w is None:
        return None, None
    q = torch.empty(w.shape, dtype=torch.uint8, device=dev())
    sc = torch.empty(w.shape[:-2] + (w.shape[-2] // 128, w.shape[-1] // 128),
                     dtype=torch.float32, device=dev())
    moe.moe_quantize_fp8(w, q, sc)
    return q, sc


def fp8_weights(moe, d):
    """Device inputs d with bf16 weights -> the same with FP8 codes + scales."""
    out = dict(d)
    for name in ("w13", "w2", "sw13", "sw2"):
        out[name], out[name + "_s"] = quantize_fp8(moe, d[name])
    torch.cuda.synchronize()
    return out


def run_layer(moe, cfg, d):
    """moe_layer_forward (or, for FP8 weights, moe_layer_forward_fp8w with
    the library's own quantization of d's weights) on device inputs d."""
    o = dict(out=empty((cfg.T, cfg.H), tdtype(cfg)), ids=empty((cfg.T, cfg.k), torch.int32),
             w=empty((cfg.T, cfg.k), torch.float32), counts=empty((cfg.E,), torch.int32),
             bal=empty((1,), torch.float32))
    ws = empty((moe.moe_workspace_size(cfg),), torch.uint8)
    if cfg.weights == "fp8":
        q = fp8_weights(moe, d)
        o["q"] = q
        call = moe.moe_layer_forward_w8a8 if cfg.acts == "fp8" else moe.moe_layer_forward_fp8w
        call(cfg, d["logits"], d["x"], q["w13"], q["w13_s"], q["w2"], q["w2_s"], q["sw13"],
             q["sw13_s"], q["sw2"], q["sw2_s"], o["out"], o["ids"], o["w"], o["counts"], o["bal"],
             ws)
    else:
        moe.moe_layer_forward(cfg, d["logits"], d["x"], d["w13"], d["w2"], d["sw13"], d["sw2"],
                              o["out"], o["ids"], o["w"], o["counts"], o["bal"], ws)
    torch.cuda.synchronize()
    # the permutation the layer built, from where it leaves it in the workspace
    off = moe.moe_layer_plan_offsets(cfg)
    S, A, R = moe.moe_num_segments(cfg), cfg.T * cfg.k, moe.moe_num_rows(cfg)
    for key, name, n in (("seg_offsets", "seg_offsets", S + 1), ("seg_expert", "seg_expert", S),
                         ("a2r", "assign_to_row", A), ("r2t", "row_to_token", R)):
        o[key] = ws[off[name]:off[name] + 4 * n].view(torch.int32).clone()
    return o


def run_permute(moe, cfg, x_d, ids_d):
    S, R = moe.moe_num_segments(cfg), moe.moe_num_rows(cfg)
    A = cfg.T * cfg.k
    o = dict(x_perm=empty((R, cfg.H), tdtype(cfg)), seg_offsets=empty((S + 1,), torch.int32),
             seg_expert=empty((S,), torch.int32), a2r=empty((A,), torch.int32),
             r2t=empty((R,), torch.int32), counts=empty((cfg.E,), torch.int32),
             bal=empty((1,), torch.float32))
    ws = empty((moe.moe_workspace_size(cfg),), torch.uint8)
    moe.moe_permute(cfg, x_d, ids_d, o["x_perm"], o["seg_offsets"], o["seg_expert"], o["a2r"],
                    o["r2t"], o["counts"], o["bal"], ws)
    torch.cuda.synchronize()
    return o


def check_plan(gpu: dict, ref: dict, n_rows: int | None = None):
    """Bit-exact permutation outputs against the oracle."""
    assert (gpu["counts"].cpu().numpy() == ref["counts"]).all(), "counts"
    assert (gpu["seg_offsets"].cpu().numpy() == ref["seg_offsets"]).all(), "seg_offsets"
    assert (gpu["seg_expert"].cpu().numpy() == ref["seg_expert"]).all(), "seg_expert"
    assert (gpu["a2r"].cpu().numpy() == ref["assign_to_row"]).all(), "assign_to_row"
    R = int(ref["seg_offsets"][-1])
    assert (gpu["r2t"].cpu().numpy()[:R] == ref["row_to_token"][:R]).all(), "row_to_token"
    assert gpu["bal"].cpu().numpy()[0] == ref["balancedness"], "balancedness"


def check_routing(cfg, ids_gpu: np.ndarray, w_gpu: np.ndarray, ids_ref, w_ref, gap,
                  logits=None):
    """ids bit-exact, except tokens whose kept-group choice sits within a few
    fp32 ulp of another (gap <= 4 ulp), where any choice among the tied groups
    is correct; there the chosen groups must all score within the tie band."""
    mism = np.nonzero((ids_gpu != ids_ref).any(axis=1))[0]
    if mism.size:
        assert cfg.score == "sigmoid", f"flat routing differs at tokens {mism[:10]}"
        gs = orc.group_scores_f32(logits[mism], cfg.n_group, cfg.group_score_topn)
        per = cfg.E // cfg.n_group
        for i, t in enumerate(mism):
            band = 4 * float(np.spacing(np.float32(np.sort(gs[i])[-cfg.topk_group])))
            assert gap[t] <= band, f"token {t}: ids differ but the group gap {gap[t]} is not a tie"
            thr = np.sort(gs[i])[-cfg.topk_group] - band
            assert all(gs[i][e // per] >= thr for e in ids_gpu[t]), f"token {t}: invalid groups"
    ok = np.setdiff1d(np.arange(cfg.T), mism)
    assert np.abs(w_gpu[ok].astype(np.float64) - w_ref[ok]).max() <= W_TOL
    return mism
