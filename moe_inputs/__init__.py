"""Seeded synthetic inputs for the single-GPU MoE layer forward.

This module only draws numbers and encodes them (fp32 -> bf16 bits by
round-to-nearest-even).  It holds none of the layer's arithmetic: no routing,
no permutation, no expert MLP.  Both the CPU oracle (tests) and the HIP path
(tests, bench) take their inputs from here, so they see the same bytes.

Streams: numpy PCG64 ``default_rng([seed, tensor_id, expert_id])`` with tensor
ids 0 logit noise, 1 popularity permutation, 2 x, 3 w13, 4 w2, 5 shared w13,
6 shared w2.  Weights are drawn per expert, so any subset of experts can be
regenerated alone (the oracle's sampled checks at full size rely on this).

Workloads (shapes from the expert-parallel serving pages: "Serving
Mixture-of-Experts Models", sections "Follow one token through an MoE layer"
and "Price one dispatch"; the Zepp paper, section 6.1 Table 2 for the
Qwen3-235B / Kimi-K2 expert shapes):

- tiny_fp32          8 tokens, hidden 256, 64 experts, top-2, I=128, fp32
- decode_bf16        64 tokens, hidden 8192, 64 experts, top-2, I=2048
- prefill_skew_bf16  4000 tokens, hidden 8192, 64 experts, top-2, I=2048,
                     Zipf(1.2) popularity bias scaled by 0.1
- deepseek_v3_bf16   4096 tokens, hidden 7168, 256 experts in 8 groups,
                     top-4 groups then top-8 (sigmoid), I=2048, + 1 shared
                     SwiGLU expert (I=2048), Zipf(1.0) bias
- ragged_stress_bf16 16384 tokens, hidden 4096, 128 experts, top-8, I=1536,
                     Zipf(1.5) bias, the 8 hottest experts split into 2
                     replica segments by token-index parity
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

T_NOISE, T_PERM, T_X, T_W13, T_W2, T_SW13, T_SW2, T_TIES = range(8)


@dataclasses.dataclass(frozen=True)
class MoEShape:
    name: str
    T: int                      # tokens
    H: int                      # hidden
    E: int                      # routed (logical) experts
    k: int                      # experts per token
    I: int                      # expert intermediate size
    dtype: str = "bf16"         # "f32" or "bf16": x, weights and outputs
    weights: str = "native"     # "native" (weights in dtype) or "fp8": the library
                                # block-quantizes the drawn bf16 weights to E4M3
    acts: str = "native"        # "fp8" (with fp8 weights): activations quantized to
                                # E4M3 in 1 x 128 pieces inside the layer (W8A8)
    score: str = "softmax"      # "softmax" (flat) or "sigmoid" (grouped)
    n_group: int = 1            # expert groups (contiguous blocks of E/n_group)
    topk_group: int = 1         # groups kept per token
    group_score_topn: int = 2   # group score = sum of its top-n member scores
    renormalize: int = 1        # weights renormalised over the k winners
    n_hot_split: int = 0        # hottest experts given replica segments
    split_ways: int = 1         # replicas per hot expert
    split_mode: str = "parity"  # "parity": replica = token index mod ways;
                                # "bounded": consecutive runs, water-filled loads
    split_c_permille: int = 0   # relaxation ratio C of the bounded split, in 1/1000
    capacity_factor_permille: int = 0   # > 0: fixed slots per expert = ceil(f * mean),
                                        # overflow dropped (masked layout)
    shared_I: int = 0           # shared expert intermediate (0 = none)
    x_std: float = 1.0
    w_std: float = 0.02
    zipf_s: float = 0.0         # popularity bias exponent (0 = none)
    zipf_alpha: float = 1.0     # scale of the log-popularity bias
    seed: int = 0

    @property
    def A(self) -> int:
        """Assignments (token, slot) pairs."""
        return self.T * self.k

    @property
    def S(self) -> int:
        """Segments: one per expert plus the extra replica segments, or kept
        rows and padding of every expert in the fixed-capacity layout."""
        if self.capacity_factor_permille > 0:
            return 2 * self.E
        return self.E + self.n_hot_split * (self.split_ways - 1)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def replace(self, **kw) -> "MoEShape":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": MoEShape("tiny_fp32", T=8, H=256, E=64, k=2, I=128, dtype="f32",
                          x_std=0.02, seed=101),
    "decode_bf16": MoEShape("decode_bf16", T=64, H=8192, E=64, k=2, I=2048, seed=102),
    "prefill_skew_bf16": MoEShape("prefill_skew_bf16", T=4000, H=8192, E=64, k=2, I=2048,
                                  zipf_s=1.2, zipf_alpha=0.1, seed=103),
    "deepseek_v3_bf16": MoEShape("deepseek_v3_bf16", T=4096, H=7168, E=256, k=8, I=2048,
                                 score="sigmoid", n_group=8, topk_group=4, group_score_topn=2,
                                 shared_I=2048, zipf_s=1.0, seed=104),
    "ragged_stress_bf16": MoEShape("ragged_stress_bf16", T=16384, H=4096, E=128, k=8, I=1536,
                                   zipf_s=1.5, n_hot_split=8, split_ways=2, seed=105),
}
# The same layers with FP8 (E4M3, 128 x 128 block-scaled) expert weights: the
# weights are drawn exactly as above and quantized by the code under test
# (the library) or by the oracle, each on its own.
for _n in ("decode", "prefill_skew", "deepseek_v3", "ragged_stress"):
    _b = WORKLOADS[_n + "_bf16"]
    WORKLOADS[_n + "_fp8w"] = dataclasses.replace(_b, name=_n + "_fp8w", weights="fp8")
    WORKLOADS[_n + "_w8a8"] = dataclasses.replace(_b, name=_n + "_w8a8", weights="fp8",
                                                  acts="fp8")
# The decode layer in the fixed-capacity (masked) layout at 1.25 x the mean
# load, overflow dropped.
WORKLOADS["decode_capacity_bf16"] = dataclasses.replace(
    WORKLOADS["decode_bf16"], name="decode_capacity_bf16", capacity_factor_permille=1250)
# The ragged layer with its hot experts split by load bounds (C = 0.1) instead
# of token parity.
WORKLOADS["ragged_stress_bounded_bf16"] = dataclasses.replace(
    WORKLOADS["ragged_stress_bf16"], name="ragged_stress_bounded_bf16", split_mode="bounded",
    split_c_permille=100)


def _rng(cfg: MoEShape, tensor_id: int, expert_id: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, tensor_id, expert_id])


# ---------------------------------------------------------------- encodings
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def values_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored input (fp32 array or bf16 bits) -> its exact float64 values."""
    if dtype == "bf16":
        return bf16_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _encode(a32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


# ---------------------------------------------------------------- logits
def popularity_bias(cfg: MoEShape) -> np.ndarray:
    """Per-expert log-popularity bias -alpha*s*ln(rank), rank a seeded
    permutation of 1..E (so the hot experts are spread over expert groups)."""
    if cfg.zipf_s == 0.0:
        return np.zeros(cfg.E, dtype=np.float64)
    rank = _rng(cfg, T_PERM).permutation(cfg.E).astype(np.float64) + 1.0
    return -cfg.zipf_alpha * cfg.zipf_s * np.log(rank)


def logits(cfg: MoEShape) -> np.ndarray:
    """Router logits fp32 [T, E]: N(0,1) noise + popularity bias, rounded to
    fp32, with every row made of distinct values (a repeated value is
    replaced by a fresh draw from the same stream until the row is distinct)."""
    rng = _rng(cfg, T_NOISE)
    noise = rng.standard_normal((cfg.T, cfg.E))
    bias = popularity_bias(cfg)
    out = (noise + bias[None, :]).astype(np.float32)
    while True:
        srt = np.sort(out, axis=1)
        dup_rows = np.nonzero((srt[:, 1:] == srt[:, :-1]).any(axis=1))[0]
        if dup_rows.size == 0:
            return out
        for t in dup_rows:
            _, first = np.unique(out[t], return_index=True)
            later = np.setdiff1d(np.arange(cfg.E), first)
            noise[t, later] = rng.standard_normal(later.size)
            out[t, later] = (noise[t, later] + bias[later]).astype(np.float32)


def tied_logits(cfg: MoEShape) -> np.ndarray:
    """Router logits fp32 [T, E] made to tie: N(0,1) draws rounded to
    multiples of 1/2 (so most rows repeat values, zero among them), about
    half of the zeros stored as -0.0, and about 2% of the entries -inf."""
    rng = _rng(cfg, T_TIES)
    out = (np.round(rng.standard_normal((cfg.T, cfg.E)) * 2.0) / 2.0).astype(np.float32)
    zero = out == 0
    neg = zero & (rng.random((cfg.T, cfg.E)) < 0.5)
    out[neg] = np.float32(-0.0)
    out[rng.random((cfg.T, cfg.E)) < 0.02] = -np.inf
    return out


# ---------------------------------------------------------------- tensors
def x(cfg: MoEShape) -> np.ndarray:
    """Token activations [T, H]: fp32 array, or uint16 bf16 bits."""
    a = _rng(cfg, T_X).standard_normal((cfg.T, cfg.H), dtype=np.float32) * np.float32(cfg.x_std)
    return _encode(a, cfg.dtype)


def w13(cfg: MoEShape, e: int) -> np.ndarray:
    """Expert e's gate and up projections, stored K-contiguous as one
    [2I, H] matrix: rows 0..I-1 are W_gate^T, rows I..2I-1 are W_up^T."""
    a = _rng(cfg, T_W13, e).standard_normal((2 * cfg.I, cfg.H), dtype=np.float32)
    return _encode(a * np.float32(cfg.w_std), cfg.dtype)


def w2(cfg: MoEShape, e: int) -> np.ndarray:
    """Expert e's down projection stored K-contiguous: [H, I] = W_down^T."""
    a = _rng(cfg, T_W2, e).standard_normal((cfg.H, cfg.I), dtype=np.float32)
    return _encode(a * np.float32(cfg.w_std), cfg.dtype)


def shared_w13(cfg: MoEShape) -> np.ndarray:
    assert cfg.shared_I > 0
    a = _rng(cfg, T_SW13).standard_normal((2 * cfg.shared_I, cfg.H), dtype=np.float32)
    return _encode(a * np.float32(cfg.w_std), cfg.dtype)


def shared_w2(cfg: MoEShape) -> np.ndarray:
    assert cfg.shared_I > 0
    a = _rng(cfg, T_SW2).standard_normal((cfg.H, cfg.shared_I), dtype=np.float32)
    return _encode(a * np.float32(cfg.w_std), cfg.dtype)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def for_each_expert(cfg: MoEShape, fn, experts=None, threads: int | None = None):
    """Calls fn(e, w13(cfg,e), w2(cfg,e)) for each expert, generating in a
    thread pool (numpy releases the GIL while drawing).  Results are yielded
    in expert order; at most ~2*threads experts are held at once."""
    experts = list(range(cfg.E)) if experts is None else list(experts)
    threads = threads or default_threads()

    def gen(e):
        return e, w13(cfg, e), w2(cfg, e)

    with ThreadPoolExecutor(max_workers=threads) as pool:
        window = 2 * threads
        futs = [pool.submit(gen, e) for e in experts[:window]]
        nxt = window
        i = 0
        while i < len(futs):
            e, a, b = futs[i].result()
            futs[i] = None
            if nxt < len(experts):
                futs.append(pool.submit(gen, experts[nxt]))
                nxt += 1
            fn(e, a, b)
            i += 1
