"""CPU oracle for the single-GPU MoE layer forward -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP product path never calls it and
shares no code with it.

It is the plain definition of what the layer computes, in float64, with numpy
library primitives (matmul, stable argsort, bincount) as single steps and no
blocking or fusion.  Sources (the pages' titles and sections):

* "Serving Mixture-of-Experts Models" (book chapter), section "Follow one token
  through an MoE layer": the router gives expert ids and weights per token; the
  runtime packs rows into contiguous per-expert segments by a histogram/sort
  over the ids (step 1), runs every expert's segment with its own row count
  (step 3), then applies the inverse permutation and a router-weighted sum
  (step 4).  Section "The slowest expert sets the pace": balancedness is mean
  load over max load, 1.0 when perfectly balanced.
* "Mixture-of-Experts Inference: parallelism, communication, and load
  balancing" (blog), section "MoE architecture recap": top-k experts per
  token from a router; grouped routing picks a few expert groups first, then
  the top experts inside them; shared experts process every token.
* Zepp paper, section 4.1: a replica changes where an expert runs, never
  which experts or weights a token gets (replica segments do not change the
  math).

Readings where the pages are silent (they are listed with reasons in the
design notes of the repository): weights are renormalised over the k winners;
slot order is descending logit (ties cannot occur: rows are distinct);
grouped routing scores experts with sigmoid, scores a group by the sum of its
top-2 member scores (computed in fp32, the precision the kernel takes that
decision in), keeps the best groups (ties to the lower group id) and then the
k largest logits inside them; the shared expert is added with weight 1;
SwiGLU is silu(x W_gate) * (x W_up) then W_down, no biases; rows inside a
segment are in increasing assignment index a = t*k + j; hot experts are the
n largest logical counts (ties to the lower id); in the parity split, replica
p of a hot expert holds the assignments whose token index t has
t mod ways == p; in the load-bounded split (Zepp section 4.1, Eq. 1 and
section 5, "Routing", restricted to one GPU) the replicas take consecutive
runs of the expert's assignments in increasing a, with loads chosen by
greedy water-filling in replica order under the integer-rounded bounds
floor(q(1-C)) <= load <= ceil(q(1+C)), q = d / ways.  With a capacity
factor f (the book's "Capacity, padding, and the drop decision"), each expert
gets ceil(f * mean) fixed slots, the assignments beyond them (in increasing
a) are dropped and contribute zero, and the rows follow the fixed-size masked
layout of the MoE inference blog ("Prefill and decode kernel layouts").

Every function here is pinned by ``tests/test_oracle_pins.py`` to facts that
do not come from this file (printed numbers, closed forms, brute force,
special cases that reduce to a dense MLP).
"""
from __future__ import annotations

from fractions import Fraction
import math

import numpy as np


# ------------------------------------------------------------------ routing
def route_flat(logits: np.ndarray, k: int, renormalize: bool = True):
    """Flat top-k gating ("MoE architecture recap": the router selects the
    top-k experts of each token).

    Returns ids int32 [T,k] in descending logit order (lower id first on an
    exact tie) and float64 weights [T,k]: softmax over the k winners, or the
    full-E softmax probability of each winner when ``renormalize`` is false.
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = l.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-l[t, e], e))[:k]
        ids[t] = order
        top = l[t, order]
        if renormalize:
            p = np.exp(top - top[0])
            w[t] = p / p.sum()
        else:
            m = l[t].max()
            w[t] = np.exp(top - m) / np.exp(l[t] - m).sum()
    return ids, w


def sigmoid_f64(l: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-np.asarray(l, dtype=np.float64)))


def group_scores_f32(logits: np.ndarray, n_group: int, topn: int) -> np.ndarray:
    """Score of each expert group: the fp32 sum, largest first, of the fp32
    sigmoid scores of its ``topn`` best members.  fp32 is the precision the
    group decision is taken in on the device as well."""
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    s32 = sigmoid_f64(l).astype(np.float32)
    gs = np.empty((T, n_group), dtype=np.float32)
    per = E // n_group
    for t in range(T):
        for g in range(n_group):
            members = sorted(s32[t, g * per:(g + 1) * per].tolist(), reverse=True)[:topn]
            acc = np.float32(0.0)
            for v in members:
                acc = np.float32(acc + np.float32(v))
            gs[t, g] = acc
    return gs


def route_grouped(logits: np.ndarray, k: int, n_group: int, topk_group: int,
                  topn: int = 2, renormalize: bool = True):
    """Group-limited routing ("MoE architecture recap": a few expert groups
    are chosen first, and the experts are then taken from inside them).

    Scores are sigmoid(logit).  Groups are contiguous blocks of E/n_group
    experts; the ``topk_group`` best groups by ``group_scores_f32`` are kept
    (lower group id on a tie); ids are the k largest logits among the kept
    groups' experts, descending.  Weights are s_j / sum(s) over the winners
    (or s_j if not renormalised), in float64.

    Also returns, per token, the fp32 gap between the last kept and the first
    dropped group score (inf if every group is kept), so that callers can tell
    which tokens sit within a few ulp of a different, equally valid choice.
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = l.shape
    per = E // n_group
    gs = group_scores_f32(logits, n_group, topn)
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    gap = np.full(T, np.inf, dtype=np.float64)
    for t in range(T):
        gorder = sorted(range(n_group), key=lambda g: (-float(gs[t, g]), g))
        kept = gorder[:topk_group]
        if topk_group < n_group:
            gap[t] = float(gs[t, gorder[topk_group - 1]]) - float(gs[t, gorder[topk_group]])
        cand = [e for g in sorted(kept) for e in range(g * per, (g + 1) * per)]
        order = sorted(cand, key=lambda e: (-l[t, e], e))[:k]
        ids[t] = order
    w = sigmoid_weights(logits, ids, renormalize)
    return ids, w, gap


def sigmoid_weights(logits: np.ndarray, ids: np.ndarray, renormalize: bool = True):
    """Weights of chosen experts in sigmoid mode: s_j = sigmoid(logit) of each
    winner, divided by their sum when renormalised (float64)."""
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    s = sigmoid_f64(np.take_along_axis(l, np.asarray(ids, dtype=np.int64), axis=1))
    return s / s.sum(axis=1, keepdims=True) if renormalize else s


# ------------------------------------------------------------------ segments
def expert_counts(ids: np.ndarray, E: int) -> np.ndarray:
    """Assignments per logical expert (the histogram of the ids)."""
    return np.bincount(np.asarray(ids).ravel(), minlength=E).astype(np.int32)


def hot_experts(counts: np.ndarray, n_hot: int) -> list:
    """The n_hot experts with the largest counts, lower id first on a tie."""
    E = len(counts)
    return sorted(range(E), key=lambda e: (-int(counts[e]), e))[:n_hot]


def segment_list(counts: np.ndarray, n_hot: int, ways: int):
    """Segments in ascending expert order; a hot expert contributes ``ways``
    adjacent replica segments (replica p first for p = 0..ways-1).

    Returns seg_expert int32 [S] and seg_replica int32 [S] (-1 = all tokens).
    """
    hot = set(hot_experts(counts, n_hot)) if n_hot > 0 and ways > 1 else set()
    seg_expert, seg_replica = [], []
    for e in range(len(counts)):
        if e in hot:
            for p in range(ways):
                seg_expert.append(e)
                seg_replica.append(p)
        else:
            seg_expert.append(e)
            seg_replica.append(-1)
    return np.array(seg_expert, dtype=np.int32), np.array(seg_replica, dtype=np.int32)


def replica_loads(d: int, ways: int, c_permille: int) -> list:
    """Per-replica loads of one hot expert with d assignments under the
    relaxed balance constraint of Zepp section 4.1, Eq. 1, on one GPU.

    The balanced reference load is q = d / ways for every replica, and
    C = c_permille / 1000 is the relaxation ratio.  Section 5 ("Routing")
    rounds the bounds to integers, floor(q(1-C)) <= load <= ceil(q(1+C)),
    and fills replicas greedily: each takes as much as its upper bound
    allows while leaving enough unassigned demand for the lower bounds of
    the replicas still to come.  All replicas live on the one GPU, so the
    source-GPU-first order of the pages is plain replica order.  Exact
    rational arithmetic."""
    q = Fraction(d, ways)
    C = Fraction(c_permille, 1000)
    lb = max(0, math.floor(q * (1 - C)))
    ub = math.ceil(q * (1 + C))
    loads, left = [], d
    for p in range(ways):
        later = ways - 1 - p
        n = min(ub, left - later * lb)
        loads.append(n)
        left -= n
    assert left == 0 and all(lb <= n <= ub for n in loads)
    return loads


def segment_of_assignments(ids: np.ndarray, seg_expert, seg_replica, ways: int,
                           loads=None) -> np.ndarray:
    """Segment of each assignment a = t*k + j.

    ``loads`` is None for the parity split (replica t mod ways), else a dict
    expert -> per-replica loads: replica p of that expert takes the
    assignments of rank loads[0] + .. + loads[p-1] up to (excluding)
    loads[0] + .. + loads[p] among the expert's assignments in increasing a.
    """
    T, k = ids.shape
    lookup = {}
    for s, (e, p) in enumerate(zip(seg_expert.tolist(), seg_replica.tolist())):
        lookup[(e, p)] = s
    seen = {}
    out = np.empty(T * k, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            s = lookup.get((e, -1))
            if s is None:
                if loads is None:
                    s = lookup[(e, t % ways)]
                else:
                    r = seen.get(e, 0)
                    seen[e] = r + 1
                    p, end = 0, loads[e][0]
                    while r >= end:
                        p += 1
                        end += loads[e][p]
                    s = lookup[(e, p)]
            out[t * k + j] = s
    return out


def permutation(seg_of_a: np.ndarray, S: int, k: int):
    """Stable counting sort of the assignments by segment ("Follow one token
    through an MoE layer", step 1).

    Returns seg_offsets int32 [S+1] (exclusive prefix sum of segment lengths),
    row_to_assign, assign_to_row and row_to_token (int32 [A]).
    """
    seg_len = np.bincount(seg_of_a, minlength=S)
    seg_offsets = np.zeros(S + 1, dtype=np.int64)
    seg_offsets[1:] = np.cumsum(seg_len)
    row_to_assign = np.argsort(seg_of_a, kind="stable")
    assign_to_row = np.empty_like(row_to_assign)
    assign_to_row[row_to_assign] = np.arange(row_to_assign.size)
    return (seg_offsets.astype(np.int32), row_to_assign.astype(np.int32),
            assign_to_row.astype(np.int32), (row_to_assign // k).astype(np.int32))


def capacity(A: int, E: int, factor_permille: int) -> int:
    """Slots per expert of the fixed-capacity layout ("Capacity, padding, and
    the drop decision"): a multiple of the mean load A / E, here
    factor = factor_permille / 1000, rounded up so that the slots hold at
    least factor x mean assignments.  Exact integer arithmetic."""
    return -(-A * factor_permille // (1000 * E))


def capacity_plan(ids: np.ndarray, E: int, cap: int):
    """The fixed-size masked layout of the MoE inference blog ("Prefill and
    decode kernel layouts") with the drop rule of the book's "Capacity,
    padding, and the drop decision": expert e owns rows [e*cap, (e+1)*cap);
    its assignments, in increasing a = t*k + j, take those rows in order, and
    the ones that find them full are dropped (assign_to_row = -1).

    Segments: 2E of them, segment 2e = expert e's kept rows, segment 2e+1 =
    its unused slots (expert -1: padding, computed by nobody).  Rows of the
    padding have row_to_token = -1.
    """
    T, k = ids.shape
    A = T * k
    used = np.zeros(E, dtype=np.int64)
    a2r = np.full(A, -1, dtype=np.int64)
    for a in range(A):
        e = int(ids[a // k, a % k])
        if not 0 <= e < E:
            continue
        if used[e] < cap:
            a2r[a] = e * cap + used[e]
        used[e] += 1
    kept = np.minimum(used, cap)
    seg_offsets = np.zeros(2 * E + 1, dtype=np.int64)
    seg_expert = np.empty(2 * E, dtype=np.int64)
    for e in range(E):
        seg_offsets[2 * e] = e * cap
        seg_offsets[2 * e + 1] = e * cap + kept[e]
        seg_expert[2 * e] = e
        seg_expert[2 * e + 1] = -1
    seg_offsets[2 * E] = E * cap
    r2a = np.full(E * cap, -1, dtype=np.int64)
    r2a[a2r[a2r >= 0]] = np.nonzero(a2r >= 0)[0]
    r2t = np.where(r2a >= 0, r2a // k, -1)
    return dict(seg_offsets=seg_offsets.astype(np.int32), seg_expert=seg_expert.astype(np.int32),
                seg_replica=np.full(2 * E, -1, dtype=np.int32),
                assign_to_row=a2r.astype(np.int32), row_to_assign=r2a.astype(np.int32),
                row_to_token=r2t.astype(np.int32), overflow=(used - kept).astype(np.int32),
                capacity=cap)


def balancedness(loads) -> np.float32:
    """mean(loads) / max(loads) ("The slowest expert sets the pace"), in
    float64, rounded once to fp32.  Zero loads count in the mean.  A batch
    with no load at all (every id dropped) has no slowest expert and the
    ratio is 0/0; it is read as 0 (the pages are silent)."""
    loads = np.asarray(loads, dtype=np.float64)
    if loads.max() == 0.0:
        return np.float32(0.0)
    return np.float32(loads.mean() / loads.max())


# ------------------------------------------------------------------ expert MLP
def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(x_rows: np.ndarray, w13_e: np.ndarray, w2_e: np.ndarray) -> np.ndarray:
    """One expert on a block of rows: silu(x W_gate) * (x W_up), then W_down.
    w13_e is [2I, H] (rows 0..I-1 = W_gate^T, I..2I-1 = W_up^T), w2_e is
    [H, I] = W_down^T; all float64."""
    I = w13_e.shape[0] // 2
    g = x_rows @ w13_e[:I].T
    u = x_rows @ w13_e[I:].T
    return (silu(g) * u) @ w2_e.T


def grouped_ffn(x_perm: np.ndarray, seg_offsets, seg_expert, w13: np.ndarray, w2: np.ndarray):
    """Every segment through its expert ("Follow one token through an MoE
    layer", step 3): y_perm rows in the permuted order, float64.  A segment
    whose expert lies outside [0, E) is padding: nothing is computed for it
    (its rows stay zero here)."""
    E = w13.shape[0]
    y = np.zeros((x_perm.shape[0], w2.shape[1]), dtype=np.float64)
    for s in range(len(seg_expert)):
        r0, r1 = int(seg_offsets[s]), int(seg_offsets[s + 1])
        e = int(seg_expert[s])
        if r1 > r0 and 0 <= e < E:
            y[r0:r1] = swiglu(x_perm[r0:r1], w13[e], w2[e])
    return y


def combine(y_perm: np.ndarray, assign_to_row, w: np.ndarray, shared_y=None):
    """Inverse permutation and router-weighted sum ("Follow one token through
    an MoE layer", step 4), plus the shared expert with weight 1.  A dropped
    assignment (row -1) contributes nothing: its output for the layer is zero
    ("Capacity, padding, and the drop decision")."""
    T, k = w.shape
    out = np.zeros((T, y_perm.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = int(assign_to_row[t * k + j])
            if r >= 0:
                out[t] += w[t, j] * y_perm[r]
    if shared_y is not None:
        out += shared_y
    return out


# ------------------------------------------------------------------ whole layer
def route(cfg, logits):
    """Routing for a workload description (fields as in moe_inputs.MoEShape)."""
    if cfg.score == "sigmoid":
        ids, w, gap = route_grouped(logits, cfg.k, cfg.n_group, cfg.topk_group,
                                    cfg.group_score_topn, bool(cfg.renormalize))
        return ids, w, gap
    ids, w = route_flat(logits, cfg.k, bool(cfg.renormalize))
    return ids, w, np.full(ids.shape[0], np.inf)


def plan(cfg, ids):
    """Histogram, segments, permutation and balancedness for routed ids."""
    counts = expert_counts(ids, cfg.E)
    cf = getattr(cfg, "capacity_factor_permille", 0)
    if cf > 0:
        p = capacity_plan(ids, cfg.E, capacity(ids.size, cfg.E, cf))
        p.update(counts=counts, balancedness=balancedness(counts))
        return p
    seg_expert, seg_replica = segment_list(counts, cfg.n_hot_split, cfg.split_ways)
    loads = None
    if getattr(cfg, "split_mode", "parity") == "bounded":
        loads = {int(e): replica_loads(int(counts[e]), cfg.split_ways, cfg.split_c_permille)
                 for e in set(seg_expert[seg_replica >= 0].tolist())}
    seg_of_a = segment_of_assignments(ids, seg_expert, seg_replica, cfg.split_ways, loads)
    seg_offsets, row_to_assign, assign_to_row, row_to_token = permutation(
        seg_of_a, len(seg_expert), cfg.k)
    return dict(counts=counts, seg_expert=seg_expert, seg_replica=seg_replica,
                seg_offsets=seg_offsets, row_to_assign=row_to_assign,
                assign_to_row=assign_to_row, row_to_token=row_to_token,
                balancedness=balancedness(counts))


def layer_forward(cfg, logits, x64, w13_64, w2_64, sw13_64=None, sw2_64=None):
    """The whole layer in float64 on small inputs: every intermediate of the
    path, keyed by name."""
    ids, w, gap = route(cfg, logits)
    p = plan(cfg, ids)
    r2t = p["row_to_token"]
    x_perm = np.where((r2t >= 0)[:, None], x64[np.maximum(r2t, 0)], 0.0)
    y_perm = grouped_ffn(x_perm, p["seg_offsets"], p["seg_expert"], w13_64, w2_64)
    shared_y = swiglu(x64, sw13_64, sw2_64) if sw13_64 is not None else None
    out = combine(y_perm, p["assign_to_row"], w, shared_y)
    p.update(ids=ids, w=w, group_gap=gap, x_perm=x_perm, y_perm=y_perm,
             shared_y=shared_y, out=out)
    return p


def token_outputs(tokens, x64_rows, ids_rows, w_rows, expert_weights, shared=None):
    """Layer output for a few tokens straight from the definition
    out[t] = sum_j w[t,j] * SwiGLU_{ids[t,j]}(x[t]) (+ shared SwiGLU(x[t])),
    for sampled checks at sizes where the whole layer is too slow.
    ``expert_weights(e)`` returns float64 (w13_e, w2_e)."""
    need = {}
    for i, _ in enumerate(tokens):
        for j, e in enumerate(ids_rows[i].tolist()):
            need.setdefault(e, []).append((i, j))
    H = x64_rows.shape[1]
    out = np.zeros((len(tokens), H), dtype=np.float64)
    for e, uses in sorted(need.items()):
        w13_e, w2_e = expert_weights(e)
        rows = np.array([i for i, _ in uses])
        y = swiglu(x64_rows[rows], w13_e, w2_e)
        for n, (i, j) in enumerate(uses):
            out[i] += w_rows[i, j] * y[n]
    if shared is not None:
        out += swiglu(x64_rows, shared[0], shared[1])
    return out
