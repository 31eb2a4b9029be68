"""Benchmark of the single-GPU MoE layer forward on one MI355X.

One step = one moe_layer_forward (route -> permute -> grouped SwiGLU ->
combine, plus balancedness) over one batch of seeded synthetic inputs that
are resident in HBM before timing starts.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline]

The default workload is the heavy-skew ragged layer (16384 tokens, hidden
4096, 128 experts, top-8, intermediate 1536), the largest single-GPU
configuration and the one bound by the matrix cores.  The roofline object is
for the grouped expert FFN (the persistent grouped-GEMM launches that
dominate the step), timed live with HIP events on the stream it runs on.
The cpu_baseline object times the float64 CPU oracle on a bounded sample of
the same workload on the host cores; practical_ceilings holds a device copy
and hipBLASLt (torch.matmul) on the same GEMM shapes, measured in the same
run outside the timed steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_inputs as mi  # noqa: E402

METRIC = "MoE-layer tokens/s and grouped-GEMM TFLOP/s (% MFMA/HBM roofline), 1 MI355X"
CSRC = os.path.join(ROOT, "mixture_experts_layer_segments_amd", "csrc")

# HBM bytes per grouped-FFN call measured with rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (summed over the dispatches of this script's grouped-FFN calls,
# per call, each counter scaled by what it reads for a plain 1 GiB device
# copy), keyed by workload.  An entry
# only applies while the library's sources (every file under csrc/) still
# hash to the value it was measured with.
MEASURED_TRAFFIC = {
    "ragged_stress_bf16": {"csrc_sha256_16": "64052207510fdc96", "bytes": 14124661746},
    "decode_bf16": {"csrc_sha256_16": "64052207510fdc96", "bytes": 5543121204},
    "prefill_skew_bf16": {"csrc_sha256_16": "64052207510fdc96", "bytes": 7615149531},
    "deepseek_v3_bf16": {"csrc_sha256_16": "64052207510fdc96", "bytes": 22227781714},
    "ragged_stress_fp8w": {"csrc_sha256_16": "64052207510fdc96", "bytes": 12672361338},
    "decode_fp8w": {"csrc_sha256_16": "64052207510fdc96", "bytes": 2776455370},
    "prefill_skew_fp8w": {"csrc_sha256_16": "64052207510fdc96", "bytes": 4219636677},
    "deepseek_v3_fp8w": {"csrc_sha256_16": "64052207510fdc96", "bytes": 14813379208},
    "ragged_stress_w8a8": {"csrc_sha256_16": "64052207510fdc96", "bytes": 7275516679},
    "decode_w8a8": {"csrc_sha256_16": "64052207510fdc96", "bytes": 2780790228},
    "prefill_skew_w8a8": {"csrc_sha256_16": "64052207510fdc96", "bytes": 3773621020},
    "deepseek_v3_w8a8": {"csrc_sha256_16": "64052207510fdc96", "bytes": 11769029962},
}


def src_hash(root=CSRC) -> str:
    """sha256 over every source file of the library (names and contents, in
    name order), first 16 hex digits."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(root)):
        path = os.path.join(root, name)
        if os.path.isfile(path) and name.endswith((".hip", ".h")):
            h.update(name.encode() + b"\0")
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    m = MEASURED_TRAFFIC.get(workload)
    if m is None or m["csrc_sha256_16"] != src_hash():
        return None
    return m["bytes"]


HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published
FP32_PEAK_TFLOPS = 157.3


# ------------------------------------------------------------------ accounting
def dispatch_bytes(cfg, assignments: int | None = None) -> int:
    """Bytes of one dispatch: one hidden-size row per assignment ("Price one
    dispatch": 2 B x hidden per routed activation; count assignments, not
    tokens)."""
    A = cfg.A if assignments is None else assignments
    return A * cfg.H * cfg.elem_bytes


def ffn_flops(cfg, rows: int | None = None) -> int:
    """Algorithmic flops of the expert MLPs: 6*H*I per computed assignment
    (gate, up and down projections; all T*k of them unless a fixed capacity
    drops some), plus 6*H*shared_I per token for a shared expert."""
    rows = cfg.A if rows is None else rows
    return 6 * cfg.H * cfg.I * rows + 6 * cfg.H * cfg.shared_I * cfg.T


def weight_bytes(cfg, n: int) -> int:
    """Bytes of n expert matrices of n x H elements: 1 byte per E4M3 code
    plus a 4-byte scale per 128 x 128 block for FP8 weights, else the
    activation element size."""
    if cfg.weights == "fp8":
        return n * cfg.H + (n * cfg.H // (128 * 128)) * 4
    return n * cfg.H * cfg.elem_bytes


def ffn_bytes(cfg, active_experts: int, rows: int | None = None) -> int:
    """Algorithmic HBM bytes of the grouped FFN: the weights of every active
    expert read once, x_perm read, h written and read, y_perm written, for
    every computed row (and the shared expert's weights and rows)."""
    eb = cfg.elem_bytes
    rows = cfg.A if rows is None else rows
    w = active_experts * weight_bytes(cfg, 3 * cfg.I)
    if cfg.acts == "fp8":
        # E4M3 x and h (1 byte + a 4-byte scale per 128), bf16 y_perm
        act = rows * (cfg.H + 2 * cfg.I + 2 * cfg.H + 4 * (cfg.H + 2 * cfg.I) // 128)
        if cfg.shared_I:
            w += weight_bytes(cfg, 3 * cfg.shared_I)
            act += cfg.T * (cfg.H + 2 * cfg.shared_I + 2 * cfg.H + 4 * (cfg.H + 2 * cfg.shared_I) // 128)
        return w + act
    act = rows * (cfg.H * 2 + cfg.I * 2) * eb
    if cfg.shared_I:
        w += weight_bytes(cfg, 3 * cfg.shared_I)
        act += cfg.T * (cfg.H * 2 + cfg.shared_I * 2) * eb
    return w + act


# ------------------------------------------------------------------ device inputs
def device_inputs(cfg):
    """Seeded inputs resident in HBM (dict of tensors)."""
    import torch
    dev = torch.device("cuda:0")
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16

    def up(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a))

    d = dict(logits=torch.from_numpy(mi.logits(cfg)).to(dev), x=up(mi.x(cfg)).to(dev))
    d["w13"] = torch.empty((cfg.E, 2 * cfg.I, cfg.H), dtype=tdt, device=dev)
    d["w2"] = torch.empty((cfg.E, cfg.H, cfg.I), dtype=tdt, device=dev)
    def put(e, a, b):
        d["w13"][e].copy_(up(a))
        d["w2"][e].copy_(up(b))

    mi.for_each_expert(cfg, put)
    d["sw13"] = d["sw2"] = None
    if cfg.shared_I:
        d["sw13"] = up(mi.shared_w13(cfg)).to(dev)
        d["sw2"] = up(mi.shared_w2(cfg)).to(dev)
    if cfg.weights == "fp8":
        # the library's block quantizer, outside any timed region; the bf16
        # weights are dropped afterwards
        import mixture_experts_layer_segments_amd as moe
        for name in ("w13", "w2", "sw13", "sw2"):
            w = d[name]
            d[name + "_s"] = None
            if w is None:
                continue
            q = torch.empty(w.shape, dtype=torch.uint8, device=dev)
            sc = torch.empty(w.shape[:-2] + (w.shape[-2] // 128, w.shape[-1] // 128),
                             dtype=torch.float32, device=dev)
            moe.moe_quantize_fp8(w, q, sc)
            d[name], d[name + "_s"] = q, sc
            del w
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    torch.cuda.synchronize()
    return d


# ------------------------------------------------------------------ cpu baseline
def cpu_baseline(cfg, logits, budget_s=20.0, min_s=10.0):
    """The float64 oracle as it stands, on the host cores: routing,
    permutation and combine of every token, and the expert MLP of active
    experts in a spread order until ~budget_s of MLP time (all of them when
    that fits).  Expert weights are regenerated and converted to float64
    outside the timed region (they are the oracle's inputs).  The MLP time
    is scaled to all active experts.  A layer whose MLPs take well under
    min_s has each expert's MLP timed several times and averaged."""
    from threadpoolctl import threadpool_limits

    from oracle import fp8 as ofp8
    from oracle import moe_oracle as orc
    threads = host_threads()
    with threadpool_limits(limits=threads):
        x64 = mi.values_f64(mi.x(cfg), cfg.dtype)
        t0 = time.perf_counter()
        ids, w, _ = orc.route(cfg, logits)
        p = orc.plan(cfg, ids)
        if cfg.acts == "fp8":          # FP8 activations: x quantized before dispatch
            x64 = ofp8.fake_quant_rows(x64)
        x_perm = x64[p["row_to_token"]]
        expert = ofp8.expert_w8a8 if cfg.acts == "fp8" else orc.swiglu
        t_route = time.perf_counter() - t0
        seg_off, seg_exp = p["seg_offsets"], p["seg_expert"]
        active_experts = np.nonzero(p["counts"] > 0)[0].tolist()
        n = len(active_experts)
        order = [active_experts[(i * 37) % n] for i in range(n)] if n % 37 else list(active_experts)
        t_ffn, done = [0.0], []
        y = np.zeros((len(p["row_to_token"]), cfg.H))

        reps = [0]

        def run(e, a, b):
            if t_ffn[0] > budget_s:
                return
            w13, w2 = mi.values_f64(a, cfg.dtype), mi.values_f64(b, cfg.dtype)
            if cfg.weights == "fp8":   # the oracle's own quantization, untimed like generation
                w13 = ofp8.dequantize_blocks(*ofp8.quantize_blocks(w13))
                w2 = ofp8.dequantize_blocks(*ofp8.quantize_blocks(w2))

            def once():
                t1 = time.perf_counter()
                for s in np.nonzero(seg_exp == e)[0]:
                    r0, r1 = int(seg_off[s]), int(seg_off[s + 1])
                    if r1 > r0:
                        y[r0:r1] = expert(x_perm[r0:r1], w13, w2)
                return time.perf_counter() - t1

            dt = once()
            if not reps[0]:
                # a layer far below min_s of CPU work is timed several times over
                reps[0] = int(min(200, max(1, np.ceil(min_s / max(dt * n, 1e-6)))))
            for _ in range(reps[0] - 1):
                dt += once()
            t_ffn[0] += dt / reps[0]
            done.append(e)

        for i in range(0, n, 8):
            if t_ffn[0] > budget_s:
                break
            # the chunk's weights are generated first (in a thread pool), so
            # that no generation runs beside the timed MLPs
            got = []
            mi.for_each_expert(cfg, lambda e, a, b: got.append((e, a, b)), experts=order[i:i + 8])
            for args_ in got:
                run(*args_)
            del got
        t0 = time.perf_counter()
        orc.combine(y, p["assign_to_row"], w)
        t_comb = time.perf_counter() - t0
    est = t_route + t_ffn[0] * n / max(1, len(done)) + t_comb
    reps_note = f", each expert MLP timed {reps[0]} times and averaged" if reps[0] > 1 else ""
    scope = ("the whole layer" + reps_note if len(done) == n else
             f"expert MLP of {len(done)} of {n} active experts ({t_ffn[0]:.1f} s), "
             f"scaled by {n}/{len(done)}")
    return {"value": cfg.T / est, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_identity(threads),
            "sample": (f"{cfg.name}: float64 numpy oracle, routing + permutation + combine of all "
                       f"{cfg.T} tokens and {scope}; {est:.2f} s per layer (weight generation"
                       f"{', FP8 quantization' if cfg.weights == 'fp8' else ''} "
                       f"and bf16->f64 conversion untimed)")}


def host_threads() -> int:
    """Threads the oracle's BLAS may use: every CPU this process may run on,
    unless the environment caps the thread pools (OMP_NUM_THREADS, which a
    shared machine may set to the process's CPU share)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_identity(threads: int) -> dict:
    """Where the oracle baseline ran: CPU model, os.cpu_count(), the threads
    used and the BLAS library numpy calls."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:  # noqa: BLE001 (identity only)
        pass
    return {"model": model, "os_cpu_count": os.cpu_count(), "threads_used": threads,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "blas": blas}


def practical_ceilings(dev, reps=10):
    """Ceilings measured in the same run, outside the timed steps: a plain
    1 GiB device copy (bytes read + written per second), a weight stream
    (torch.matmul in bf16, hipBLASLt, of 64 rows by a 1 GiB weight, 8192 x
    65536: weight bytes read per second, the decode layers' regime) and
    torch.matmul in bf16 on the ragged layer's two dense GEMM shapes."""
    import torch
    out = {}
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    out["device_copy_1GiB_GBs"] = round(2 * (1 << 30) / (ms * 1e-3) / 1e9, 1)
    del src, dst
    a = torch.randn((64, 8192), dtype=torch.bfloat16, device=dev)
    wt = torch.randn((8192, 65536), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.matmul(a, wt)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(a, wt)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    out["matmul_bf16_64x65536x8192_weight_GBs"] = round(wt.numel() * 2 / (ms * 1e-3) / 1e9, 1)
    del a, wt
    for m_, n_, k_ in ((16384, 3072, 4096), (16384, 4096, 1536)):
        a = torch.randn((m_, k_), dtype=torch.bfloat16, device=dev)
        b = torch.randn((k_, n_), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"matmul_bf16_{m_}x{n_}x{k_}_TFLOPs"] = round(2 * m_ * n_ * k_ / (ms * 1e-3) / 1e12, 1)
        del a, b
    torch.cuda.empty_cache()
    return out


def calibrate_copy(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, so that HBM counters (FETCH_SIZE,
    WRITE_SIZE) can be scaled: each copy reads and writes `nbytes`."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": nbytes,
                      "bytes_written_per_copy": nbytes, "copies": reps}), flush=True)
    return 0


# ------------------------------------------------------------------ main
def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ragged_stress_bf16", choices=sorted(mi.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the device-copy and torch.matmul ceilings (profiling runs)")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="run the timed steps as eager calls, or as replays of one HIP graph "
                         "captured from a step (the other mode is timed too and reported)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args(argv)
    if args.calibrate_copy:
        return calibrate_copy()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by expert parallelism across GPUs, which is not built here)",
              file=sys.stderr)
        return 2

    import torch

    import mixture_experts_layer_segments_amd as moe
    cfg = mi.WORKLOADS[args.workload]
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    d = device_inputs(cfg)

    dev = torch.device("cuda:0")
    tdt = d["x"].dtype
    out = torch.empty((cfg.T, cfg.H), dtype=tdt, device=dev)
    ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    counts = torch.empty((cfg.E,), dtype=torch.int32, device=dev)
    bal = torch.empty((1,), dtype=torch.float32, device=dev)
    ws = torch.empty((moe.moe_workspace_size(cfg),), dtype=torch.uint8, device=dev)

    fp8 = cfg.weights == "fp8"
    w8a8 = cfg.acts == "fp8"
    xq = xs = None          # W8A8: x_perm quantized for the FFN leg (outside its timing)

    def step():
        if w8a8:
            moe.moe_layer_forward_w8a8(cfg, d["logits"], d["x"], d["w13"], d["w13_s"], d["w2"],
                                       d["w2_s"], d["sw13"], d["sw13_s"], d["sw2"], d["sw2_s"],
                                       out, ids, w, counts, bal, ws)
        elif fp8:
            moe.moe_layer_forward_fp8w(cfg, d["logits"], d["x"], d["w13"], d["w13_s"], d["w2"],
                                       d["w2_s"], d["sw13"], d["sw13_s"], d["sw2"], d["sw2_s"],
                                       out, ids, w, counts, bal, ws)
        else:
            moe.moe_layer_forward(cfg, d["logits"], d["x"], d["w13"], d["w2"], d["sw13"],
                                  d["sw2"], out, ids, w, counts, bal, ws)

    def ffn():
        if w8a8:
            moe.moe_grouped_ffn_w8a8(cfg, xq, xs, so, se, d["w13"], d["w13_s"], d["w2"],
                                     d["w2_s"], None, y_perm, ws)
        elif fp8:
            moe.moe_grouped_ffn_fp8w(cfg, x_perm, so, se, d["w13"], d["w13_s"], d["w2"],
                                     d["w2_s"], None, y_perm, ws)
        else:
            moe.moe_grouped_ffn(cfg, x_perm, so, se, d["w13"], d["w2"], None, y_perm, ws)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # One step captured into a HIP graph: every grid depends only on the
    # configuration (segment lengths stay on the device), so replays serve
    # any routing.
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()

    def timed(run):
        """Mean over exactly K steps (events around all of them), and the
        median and min of per-step events recorded between the steps.  W
        untimed runs of the same kind come right before them: after the host
        has waited, the first steps run at a lower clock while it ramps up."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(args.steps):
            run()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
        return (ev[0].elapsed_time(ev[-1]) / args.steps, time.perf_counter() - t0,
                float(np.median(per)), float(per.min()))

    ms_eager, wall_eager, med_eager, min_eager = timed(step)
    ms_graph, wall_graph, med_graph, min_graph = timed(graph.replay)
    if args.launch == "graph":
        ms, wall, med, mn = ms_graph, wall_graph, med_graph, min_graph
    else:
        ms, wall, med, mn = ms_eager, wall_eager, med_eager, min_eager
    counts_h = counts.cpu().numpy()
    active = int((counts_h > 0).sum())   # experts whose weights the step must read
    cap = moe.moe_num_rows(cfg) // cfg.E if cfg.capacity_factor_permille else cfg.A
    computed = int(np.minimum(counts_h, cap).sum())   # rows the FFN computes (drops excluded)

    # dominant kernels: the grouped FFN on the permuted rows of this batch
    S, R = moe.moe_num_segments(cfg), moe.moe_num_rows(cfg)
    A = cfg.A
    x_perm = torch.empty((R, cfg.H), dtype=tdt, device=dev)
    y_perm = torch.empty((R, cfg.H), dtype=tdt, device=dev)
    so = torch.empty((S + 1,), dtype=torch.int32, device=dev)
    se = torch.empty((S,), dtype=torch.int32, device=dev)
    a2r = torch.empty((A,), dtype=torch.int32, device=dev)
    r2t = torch.empty((R,), dtype=torch.int32, device=dev)
    moe.moe_permute(cfg, d["x"], ids, x_perm, so, se, a2r, r2t, counts, bal, ws)
    if w8a8:
        xq = torch.empty((R, cfg.H), dtype=torch.uint8, device=dev)
        xs = torch.empty((R, cfg.H // 128), dtype=torch.float32, device=dev)
        moe.moe_quantize_act_fp8(x_perm, xq, xs)
    ffn_ms, _, ffn_med, ffn_min = timed(ffn)

    routed = cfg.replace(shared_I=0)
    fl = ffn_flops(routed, computed)
    by = ffn_bytes(routed, active, computed)
    gbs = by / (ffn_ms * 1e-3) / 1e9
    tflops = fl / (ffn_ms * 1e-3) / 1e12
    mfma_peak = FP8_PEAK_TFLOPS if w8a8 else BF16_PEAK_TFLOPS   # the contraction's own dtype
    hbm_bound = fl / (mfma_peak * 1e12) < by / (HBM_PEAK_GBS * 1e9)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(cfg.name)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(tflops / mfma_peak, 4),
                "traffic": measured_traffic(cfg.name)}
    roof["kernel"] = ("grouped FFN: the grouped-GEMM launches of one moe_grouped_ffn"
                      + ("_w8a8" if w8a8 else "_fp8w" if fp8 else "")
                      + " call (GEMM 1 gate/up + SwiGLU, then GEMM 2 down + row scale; each "
                        "one launch per tile shape)")
    roof["ms_per_launch"] = round(ffn_ms, 4)
    roof["ms_per_launch_median"] = round(ffn_med, 4)
    roof["ms_per_launch_min"] = round(ffn_min, 4)
    roof["traffic_source"] = ("rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on these sources "
                              f"(csrc sha256 {src_hash()})" if roof["traffic"] is not None else
                              "not measured for the current sources")
    roof["algorithmic_bytes"] = by
    roof["algorithmic_flops"] = fl

    res = {
        "metric": METRIC, "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "ms_per_step_median": round(med, 4),
        "ms_per_step_min": round(mn, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3" if w8a8 else cfg.dtype,
        "data": "synthetic (seeded; random-init weights)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "experts": cfg.E,
                   "top_k": cfg.k, "intermediate": cfg.I, "shared_intermediate": cfg.shared_I,
                   "assignments": cfg.A, "active_experts": active,
                   "weights": ("fp8 e4m3, 128x128 power-of-two block scales" +
                               ("" if w8a8 else ", dequantized to bf16 in the GEMMs"))
                   if fp8 else cfg.dtype,
                   **({"activations": "fp8 e4m3, 1x128 power-of-two scales (x before dispatch, "
                                      "h between the GEMMs); fp8 x fp8 MFMAs"} if w8a8 else {}),
                   "balancedness": float(bal.item()),
                   **({"capacity_factor": cfg.capacity_factor_permille / 1000,
                       "slots_per_expert": cap, "computed_assignments": computed}
                      if cfg.capacity_factor_permille else {}),
                   **({"split": cfg.split_mode, "split_c": cfg.split_c_permille / 1000}
                      if cfg.n_hot_split else {})},
        "grouped_gemm_tflops": round(tflops, 2),
        "grouped_gemm_frac_mfma": round(tflops / mfma_peak, 4),
        "grouped_gemm_frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
        "wall_s_timed": round(wall, 3),
        "launch": args.launch,
        "ms_per_step_eager": round(ms_eager, 4),
        "ms_per_step_graph_replay": round(ms_graph, 4),
        "roofline": roof,
    }
    if not args.no_ceilings:
        print("[bench] practical ceilings", file=sys.stderr, flush=True)
        res["practical_ceilings"] = practical_ceilings(dev)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, mi.logits(cfg))
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
