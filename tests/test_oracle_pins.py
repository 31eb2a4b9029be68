"""Pins for the CPU oracle: facts that do not come from the oracle itself.

Each test names the passage or the mathematical fact it checks; each is
chosen so that a plausible slip in the oracle (a dropped term, a wrong sign
or index, a transposed operand, a wrong inverse) fails at least one of them.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special

import moe_inputs as mi
from oracle import moe_oracle as o

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _distinct_logits(rng, T, E):
    while True:
        l = rng.standard_normal((T, E)).astype(np.float32)
        if all(len(set(r.tolist())) == E for r in l):
            return l


def _tiny(T=24, H=16, E=6, k=2, I=8, **kw):
    cfg = mi.MoEShape("pin", T=T, H=H, E=E, k=k, I=I, dtype="f32", **kw)
    rng = np.random.default_rng(7)
    lg = _distinct_logits(rng, T, E)
    x = rng.standard_normal((T, H))
    w13 = rng.standard_normal((E, 2 * I, H)) * 0.3
    w2 = rng.standard_normal((E, H, I)) * 0.3
    return cfg, lg, x, w13, w2


# ---------------------------------------------------------------- printed facts
def test_token_flow_printed_example():
    """8 tokens, 64 experts, top-2 -> 16 expert executions, 16 outputs
    combined into 8 ("Follow one token through an MoE layer")."""
    g = _gold("serving_moe_token_flow.json")["token_flow"]
    cfg = mi.WORKLOADS["tiny_fp32"]
    assert (cfg.T, cfg.E, cfg.k) == (g["tokens"], g["experts"], g["top_k"])
    lg = mi.logits(cfg)
    x = mi.values_f64(mi.x(cfg), cfg.dtype)
    E, I, H = cfg.E, cfg.I, cfg.H
    rng = np.random.default_rng(0)
    w13 = rng.standard_normal((E, 2 * I, H)) * 0.02
    w2 = rng.standard_normal((E, H, I)) * 0.02
    r = o.layer_forward(cfg, lg, x, w13, w2)
    assert r["ids"].size == g["expert_executions"]
    assert r["y_perm"].shape[0] == g["expert_executions"]
    assert r["out"].shape[0] == g["outputs_combined_into"]
    assert int(r["seg_offsets"][-1]) == 16
    # each token uses about 3% of the expert weights (book, "Follow one token
    # through an MoE layer")
    assert abs(cfg.k / cfg.E - _gold("serving_moe_token_flow.json")["expert_fraction_per_token_approx"]) < 0.005


def test_balancedness_worked_example():
    """Counts 22,14,7,6,5,4,3,3 on 4 ranks of 2 contiguous experts: loads
    36,13,9,6, mean 16, balancedness 16/36 ~ 0.44; the repack gives max 25
    ("Worked example: balance the busiest rank")."""
    g = _gold("serving_moe_worked_example.json")
    counts = np.array(g["expert_counts"])
    per = g["experts_per_rank"]
    loads = counts.reshape(-1, per).sum(axis=1)
    assert loads.tolist() == g["rank_loads"]
    b = o.balancedness(loads)
    num, den = g["balancedness_per_rank_exact"]
    assert b == np.float32(num / den)
    assert round(float(b), 2) == g["balancedness_per_rank_approx"]
    repacked = [counts[list(p)].sum() for p in g["repacked_pairs"]]
    assert repacked == g["repacked_rank_loads"]
    assert o.balancedness(repacked) == np.float32(16 / 25)
    # per logical expert (the unit used for one layer on one GPU): 8/22
    assert o.balancedness(counts) == np.float32(8 / 22)
    assert o.balancedness(o.expert_counts(np.repeat(np.arange(8), 8), 8)) == g["perfect_balance"]


def test_uniform_routing_balancedness_is_one():
    """Balancedness is 1.0 when every expert carries the same load ("The
    slowest expert sets the pace"): token t routed to experts 2t mod E and
    2t+1 mod E."""
    T, E, k = 64, 16, 2
    lg = np.empty((T, E), dtype=np.float32)
    for t in range(T):
        lg[t] = -np.arange(E, dtype=np.float32) / 100.0 - 1.0
        lg[t, (2 * t) % E] = 5.0
        lg[t, (2 * t + 1) % E] = 4.0
    ids, _ = o.route_flat(lg, k)
    assert all(ids[t].tolist() == [(2 * t) % E, (2 * t + 1) % E] for t in range(T))
    c = o.expert_counts(ids, E)
    assert (c == T * k // E).all()
    assert o.balancedness(c) == np.float32(1.0)


@pytest.mark.parametrize("seed", range(6))
def test_balancedness_is_a_fraction_and_scale_free(seed):
    """For any loads with a positive maximum, mean/max lies in [1/E, 1]: it is
    1/E exactly when one expert holds everything, and it does not change when
    every load is multiplied by the same factor.  With no load at all (every
    id dropped) the ratio is 0/0 and reads as 0, below every defined value, so
    an empty batch never looks balanced."""
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 40))
    c = rng.integers(0, 50, size=E)
    c[rng.integers(0, E)] += 1
    b = float(o.balancedness(c))
    assert 1.0 / E - 1e-7 <= b <= 1.0
    assert o.balancedness(3 * c) == o.balancedness(c)
    one = np.zeros(E, dtype=np.int64)
    one[rng.integers(0, E)] = 7
    assert o.balancedness(one) == np.float32(1.0 / E)
    assert o.balancedness(np.zeros(E, dtype=np.int64)) == np.float32(0.0)


def test_empty_experts_are_normal():
    """An expert may get no token at all (Zepp section 2): its segment stays in
    the list with length 0 and the mean still counts it."""
    cfg, lg, x, w13, w2 = _tiny(T=4, E=12, k=1)
    r = o.layer_forward(cfg, lg, x, w13, w2)
    lens = np.diff(r["seg_offsets"])
    assert len(lens) == 12 and (lens == 0).sum() >= 8
    assert r["balancedness"] == np.float32((4 / 12) / r["counts"].max())


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("E,k,seed", [(5, 1, 0), (6, 2, 1), (9, 3, 2), (12, 4, 3), (7, 7, 4)])
def test_route_flat_brute_force(E, k, seed):
    """The chosen set maximises the sum of logits over all C(E,k) subsets
    (unique: values are distinct); slots are in descending logit order."""
    rng = np.random.default_rng(seed)
    lg = _distinct_logits(rng, 10, E)
    ids, w = o.route_flat(lg, k)
    for t in range(10):
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(float(lg[t, e]) for e in c))
        assert set(ids[t].tolist()) == set(best)
        vals = lg[t, ids[t]]
        assert all(vals[j] > vals[j + 1] for j in range(k - 1))
        # softmax over the winners: ratios exp(l_i - l_j), sum 1
        assert abs(w[t].sum() - 1.0) < 1e-15
        for i in range(k):
            for j in range(k):
                assert np.isclose(w[t, i] / w[t, j], np.exp(float(vals[i]) - float(vals[j])), rtol=1e-13)


def test_route_flat_k2_closed_form():
    """k = 2: w0 = 1 / (1 + exp(l1 - l0))."""
    lg = _distinct_logits(np.random.default_rng(11), 50, 64)
    ids, w = o.route_flat(lg, 2)
    l0 = lg[np.arange(50), ids[:, 0]].astype(np.float64)
    l1 = lg[np.arange(50), ids[:, 1]].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], scipy.special.expit(l0 - l1), rtol=1e-14)


def test_route_flat_without_renormalising_is_full_softmax():
    lg = _distinct_logits(np.random.default_rng(12), 20, 10)
    ids, w = o.route_flat(lg, 3, renormalize=False)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-13)


def test_route_grouped_brute_force():
    """E=16 in 4 groups, keep 2 groups, top-3: enumerate every group pair by
    the sum of its group scores (score = sum of the 2 best member sigmoids),
    then every 3-subset of the pair's experts."""
    rng = np.random.default_rng(5)
    lg = _distinct_logits(rng, 40, 16)
    ids, w, gap = o.route_grouped(lg, 3, n_group=4, topk_group=2, topn=2)
    s = scipy.special.expit(lg.astype(np.float64))
    for t in range(40):
        gsc = [sum(sorted(s[t, 4 * g:4 * g + 4])[-2:]) for g in range(4)]
        pair = max(itertools.combinations(range(4), 2), key=lambda p: gsc[p[0]] + gsc[p[1]])
        members = [e for g in pair for e in range(4 * g, 4 * g + 4)]
        best = max(itertools.combinations(members, 3), key=lambda c: sum(float(lg[t, e]) for e in c))
        assert set(ids[t].tolist()) == set(best), t
        assert list(lg[t, ids[t]]) == sorted(lg[t, ids[t]], reverse=True)
        np.testing.assert_allclose(w[t], s[t, ids[t]] / s[t, ids[t]].sum(), rtol=1e-14)
        assert gap[t] > 0


def test_route_grouped_one_group_is_flat_sigmoid_topk():
    lg = _distinct_logits(np.random.default_rng(6), 30, 24)
    ids_g, w_g, _ = o.route_grouped(lg, 5, n_group=1, topk_group=1)
    ids_f, _ = o.route_flat(lg, 5)
    assert (ids_g == ids_f).all()
    s = scipy.special.expit(lg.astype(np.float64))
    sel = np.take_along_axis(s, ids_f.astype(np.int64), 1)
    np.testing.assert_allclose(w_g, sel / sel.sum(1, keepdims=True), rtol=1e-14)


def test_sigmoid_weights_of_given_ids():
    """The weights of any chosen ids (used where the GPU's group choice sits
    on a tie): sigmoid of each winner's logit (scipy's expit), divided by
    their sum when renormalised; for the routed ids they are route_grouped's."""
    rng = np.random.default_rng(7)
    lg = _distinct_logits(rng, 25, 32)
    ids = np.stack([rng.permutation(32)[:4] for _ in range(25)]).astype(np.int32)
    s = np.take_along_axis(scipy.special.expit(lg.astype(np.float64)), ids.astype(np.int64), 1)
    np.testing.assert_allclose(o.sigmoid_weights(lg, ids, False), s, rtol=1e-14)
    np.testing.assert_allclose(o.sigmoid_weights(lg, ids), s / s.sum(1, keepdims=True), rtol=1e-14)
    ids_g, w_g, _ = o.route_grouped(lg, 4, n_group=4, topk_group=2)
    assert np.array_equal(o.sigmoid_weights(lg, ids_g), w_g)


def test_group_scores_are_fp32_sums_of_best_members():
    """fp32 group scores lie within 2 ulp of the exact top-2 sigmoid sums."""
    lg = _distinct_logits(np.random.default_rng(8), 16, 64)
    gs = o.group_scores_f32(lg, 8, 2)
    s = scipy.special.expit(lg.astype(np.float64))
    for t in range(16):
        for g in range(8):
            exact = sum(sorted(s[t, 8 * g:8 * g + 8])[-2:])
            assert abs(float(gs[t, g]) - exact) <= 2 * np.spacing(np.float32(exact))


# ---------------------------------------------------------------- permutation
def _counting_sort_rows(seg_of_a, S):
    rows = []
    for s in range(S):
        for a in range(len(seg_of_a)):
            if seg_of_a[a] == s:
                rows.append(a)
    return np.array(rows)


@pytest.mark.parametrize("T,E,k,hot,ways", [(24, 6, 2, 0, 1), (37, 8, 3, 2, 2), (50, 5, 5, 0, 1), (33, 9, 2, 3, 3)])
def test_permutation_is_stable_bijection(T, E, k, hot, ways):
    """Rows of a segment are its assignments in increasing a = t*k+j; the
    permutation is a bijection; segment lengths merge back to the expert
    histogram ("Follow one token through an MoE layer", step 1)."""
    cfg, lg, x, w13, w2 = _tiny(T=T, E=E, k=k, n_hot_split=hot, split_ways=ways)
    r = o.layer_forward(cfg, lg, x, w13, w2)
    A = T * k
    r2a, a2r = r["row_to_assign"], r["assign_to_row"]
    assert sorted(r2a.tolist()) == list(range(A))
    assert (a2r[r2a] == np.arange(A)).all()
    S = len(r["seg_expert"])
    seg_of_a = o.segment_of_assignments(r["ids"], r["seg_expert"], r["seg_replica"], ways)
    assert (r2a == _counting_sort_rows(seg_of_a.tolist(), S)).all()
    lens = np.diff(r["seg_offsets"])
    merged = np.zeros(E, dtype=np.int64)
    np.add.at(merged, r["seg_expert"], lens)
    assert (merged == np.bincount(r["ids"].ravel(), minlength=E)).all()
    assert (r["row_to_token"] == r2a // k).all()
    assert (r["x_perm"] == x[r["row_to_token"]]).all()
    # every row of a segment really belongs to that segment's expert
    for s in range(S):
        for row in range(r["seg_offsets"][s], r["seg_offsets"][s + 1]):
            a = r2a[row]
            assert r["ids"][a // k, a % k] == r["seg_expert"][s]
            if r["seg_replica"][s] >= 0:
                assert (a // k) % ways == r["seg_replica"][s]


def test_hot_experts_are_the_largest_counts():
    counts = np.array([5, 9, 9, 1, 0, 9, 3, 7])
    assert o.hot_experts(counts, 3) == [1, 2, 5]
    assert o.hot_experts(counts, 4) == [1, 2, 5, 7]
    se, sr = o.segment_list(counts, 2, 2)
    assert se.tolist() == [0, 1, 1, 2, 2, 3, 4, 5, 6, 7]
    assert sr.tolist() == [-1, 0, 1, 0, 1, -1, -1, -1, -1, -1]


# ------------------------------------------------- load-bounded replica split
def _feasible(d, ways, c_permille):
    """Every integer load vector of the rounded relaxed-balance bounds of
    Zepp section 4.1, Eq. 1 (with the integer rounding of section 5,
    "Routing"), by brute force, in lexicographic order."""
    q_num, q_den = d * (1000 - c_permille), 1000 * ways         # q(1-C) as a fraction
    lb = max(0, q_num // q_den) if c_permille <= 1000 else 0
    ub = -((-d * (1000 + c_permille)) // q_den)                 # ceil(q(1+C))
    out = []
    for n in itertools.product(range(d + 1), repeat=ways):
        if sum(n) == d and all(lb <= v <= ub for v in n):
            out.append(list(n))
    return out, lb, ub


@pytest.mark.parametrize("ways,c", [(2, 0), (2, 250), (3, 0), (3, 500), (3, 1500), (4, 100)])
def test_water_filling_is_the_greediest_feasible_split(ways, c):
    """Brute force over all load vectors: the bounds admit at least one, the
    oracle's loads are one of them, and greedy filling in replica order
    (each replica as full as the others' lower bounds allow) is the
    lexicographically largest feasible vector."""
    for d in range(0, 19):
        feas, lb, ub = _feasible(d, ways, c)
        got = o.replica_loads(d, ways, c)
        assert feas, (d, ways, c)
        assert got in feas, (d, ways, c, got, lb, ub)
        assert got == max(feas), (d, ways, c, got, max(feas))


def test_water_filling_closed_forms():
    """C = 0: the near-equal split of d into ways parts, larger parts first
    (numpy's array_split sizes); C >= ways - 1: the upper bound reaches d and
    the lower bound is 0, so replica 0 takes all; integer q with C = 0: every
    replica gets exactly q."""
    for d in range(0, 40):
        for ways in (2, 3, 4):
            sizes = [len(part) for part in np.array_split(np.arange(d), ways)]
            assert o.replica_loads(d, ways, 0) == sizes
            assert o.replica_loads(d, ways, 1000 * (ways - 1)) == [d] + [0] * (ways - 1)
    assert o.replica_loads(12, 3, 0) == [4, 4, 4]
    assert o.replica_loads(10, 3, 500) == [5, 4, 1]     # q = 10/3: bounds 1 .. 5
    assert o.replica_loads(100, 2, 250) == [63, 37]     # q = 50: bounds 37 .. 63


@pytest.mark.parametrize("c", [0, 300, 1000])
def test_bounded_split_only_moves_segment_boundaries(c):
    """The bounded split cuts each hot expert's rows, in increasing a, into
    consecutive runs: the row order equals the unsplit permutation's, the
    runs have the water-filled lengths, every row belongs to its segment's
    expert, and the layer output is bit for bit the unsplit one (replicas
    keep the logical selection and weights, Zepp section 4.1)."""
    cfg, lg, x, w13, w2 = _tiny(T=47, E=6, k=3, n_hot_split=2, split_ways=3,
                                split_mode="bounded", split_c_permille=c)
    a = o.layer_forward(cfg, lg, x, w13, w2)
    b = o.layer_forward(cfg.replace(n_hot_split=0, split_ways=1, split_mode="parity"), lg, x,
                        w13, w2)
    assert (a["row_to_assign"] == b["row_to_assign"]).all()
    assert (a["out"] == b["out"]).all()
    counts = np.bincount(a["ids"].ravel(), minlength=cfg.E)
    hot = sorted(range(cfg.E), key=lambda e: (-counts[e], e))[:2]
    lens = np.diff(a["seg_offsets"])
    for e in range(cfg.E):
        mine = np.nonzero(a["seg_expert"] == e)[0]
        if e in hot:
            d = int(counts[e])
            assert len(mine) == 3
            # the brute-force greediest feasible vector, independent of the oracle
            assert lens[mine].tolist() == max(_feasible(d, 3, c)[0])
        else:
            assert lens[mine].tolist() == [counts[e]]
        rows = a["row_to_assign"][a["seg_offsets"][mine[0]]:a["seg_offsets"][mine[-1] + 1]]
        assert (a["ids"].ravel()[rows] == e).all() and (np.diff(rows) > 0).all()


# ------------------------------------------------- capacity and drop
def _ids_with_counts(counts, k):
    """[T, k] ids with the given per-expert counts and distinct experts per
    token: the assignments sorted by expert, slot j of token t taking item
    j*T + t (T >= the largest count keeps a token's experts distinct)."""
    items = np.repeat(np.arange(len(counts)), counts)
    T = len(items) // k
    assert T >= max(counts)
    ids = items.reshape(k, T).T.copy()
    assert all(len(set(r.tolist())) == k for r in ids)
    return ids


def test_capacity_worked_example():
    """1.25 x the mean of 8 gives 10 slots per expert (80 in all) for the 64
    assignments, and expert 0 (22 assignments) overflows by 12; sizing every
    expert for the busiest gives 22 x 8 = 176 slots, about two thirds of them
    padding ("Capacity, padding, and the drop decision")."""
    g = _gold("serving_moe_capacity.json")
    counts = g["expert_counts"]
    E, A = len(counts), g["assignments"]
    assert A == sum(counts) and A / E == g["mean_per_expert"]
    cap = o.capacity(A, E, round(g["capacity_factor"] * 1000))
    assert cap == g["slots_per_expert"] and E * cap == g["total_slots"]
    ids = _ids_with_counts(counts, 2)
    p = o.capacity_plan(ids, E, cap)
    assert p["overflow"][0] == g["expert0_overflow"]
    assert p["overflow"].tolist() == [max(0, c - cap) for c in counts]
    # padding to the maximum: the factor max / mean drops nothing
    cap_max = o.capacity(A, E, 2750)             # factor 22 / 8 = 2.75
    assert cap_max == g["pad_to_max_slots_per_expert"]
    assert E * cap_max == g["pad_to_max_total_slots"]
    assert abs((E * cap_max - A) / (E * cap_max) - g["pad_to_max_padding_fraction_approx"]) < 0.04
    assert not o.capacity_plan(ids, E, cap_max)["overflow"].any()


def test_capacity_rounds_up_to_hold_factor_times_mean():
    assert o.capacity(63, 8, 1250) == 10        # 9.84 slots needed -> 10
    assert o.capacity(64, 8, 1000) == 8
    assert o.capacity(65, 8, 1000) == 9
    assert o.capacity(1, 64, 1) == 1


@pytest.mark.parametrize("cap", [1, 3, 10])
def test_masked_layout_and_drop_rule_by_brute_force(cap):
    """Expert e owns rows [e*cap, (e+1)*cap); its first cap assignments in
    increasing a fill them in order, the rest are dropped (row -1); the
    segments are [kept rows of e, padding of e] for every e."""
    counts = [22, 14, 7, 6, 5, 4, 3, 3]
    ids = _ids_with_counts(counts, 2)
    E, k = len(counts), 2
    p = o.capacity_plan(ids, E, cap)
    flat = ids.ravel()
    for e in range(E):
        mine = [a for a in range(flat.size) if flat[a] == e]
        for n, a in enumerate(mine):
            assert p["assign_to_row"][a] == (e * cap + n if n < cap else -1)
        kept = min(len(mine), cap)
        assert p["seg_offsets"][2 * e] == e * cap and p["seg_offsets"][2 * e + 1] == e * cap + kept
        assert p["seg_expert"][2 * e] == e and p["seg_expert"][2 * e + 1] == -1
        assert (p["row_to_token"][e * cap + kept:(e + 1) * cap] == -1).all()
    assert p["seg_offsets"][-1] == E * cap


def test_capacity_layer_drops_exactly_the_overflow():
    """The layer with a capacity equals the definition with the dropped
    slots' terms removed (their outputs become zeros); a capacity that holds
    every assignment gives the dropless layer."""
    cfg, lg, x, w13, w2 = _tiny(T=40, E=6, k=3, zipf_s=1.2)
    free = o.layer_forward(cfg, lg, x, w13, w2)
    roomy = o.layer_forward(cfg.replace(capacity_factor_permille=2000), lg, x, w13, w2)
    assert roomy["capacity"] == 40 and (roomy["assign_to_row"] >= 0).all()   # 2 x mean 20
    np.testing.assert_allclose(roomy["out"], free["out"], rtol=1e-12, atol=1e-13)
    tight = o.layer_forward(cfg.replace(capacity_factor_permille=900), lg, x, w13, w2)
    cap = tight["capacity"]
    assert cap == -(-40 * 3 * 900 // (1000 * 6))
    ids, w = free["ids"], free["w"]
    seen, keep = {}, np.zeros(ids.shape, dtype=bool)
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            keep[t, j] = seen.get(e, 0) < cap
            seen[e] = seen.get(e, 0) + 1
    assert not keep.all()
    want = o.token_outputs(list(range(40)), x, ids, np.where(keep, w, 0.0),
                           lambda e: (w13[e], w2[e]))
    np.testing.assert_allclose(tight["out"], want, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- expert MLP
def test_swiglu_hand_example():
    """x = [1, 2]; W_gate column [0.5, 0.25] -> g = 1; W_up column [1, -1]
    -> u = -1; h = silu(1) * -1 = -1/(1+e^-1); W_down row [2, 3]."""
    x = np.array([[1.0, 2.0]])
    w13 = np.array([[0.5, 0.25], [1.0, -1.0]])       # [2I=2, H=2]
    w2 = np.array([[2.0], [3.0]])                      # [H=2, I=1]
    h = -0.7310585786300049                            # -sigmoid(1)
    np.testing.assert_allclose(o.swiglu(x, w13, w2), [[2 * h, 3 * h]], rtol=1e-15)
    assert o.silu(np.array([0.0]))[0] == 0.0
    assert o.silu(np.array([-800.0]))[0] == 0.0
    assert o.silu(np.array([40.0]))[0] == 40.0


def _dense(x, w13, w2):
    I = w13.shape[0] // 2
    g = x @ w13[:I].T
    return (g * scipy.special.expit(g) * (x @ w13[I:].T)) @ w2.T


def test_identical_experts_reduce_to_dense_mlp():
    """With every expert equal and weights renormalised, the routed layer is
    the dense SwiGLU MLP: routing, permutation and combine cancel out."""
    cfg, lg, x, w13, w2 = _tiny(T=31, E=7, k=3, n_hot_split=2, split_ways=2)
    w13[:] = w13[0]
    w2[:] = w2[0]
    r = o.layer_forward(cfg, lg, x, w13, w2)
    np.testing.assert_allclose(r["out"], _dense(x, w13[0], w2[0]), rtol=1e-12, atol=1e-12)


def test_one_expert_top1_is_dense_mlp():
    cfg, lg, x, w13, w2 = _tiny(T=9, E=1, k=1)
    r = o.layer_forward(cfg, lg, x, w13, w2)
    assert (r["w"] == 1.0).all()
    np.testing.assert_allclose(r["out"], _dense(x, w13[0], w2[0]), rtol=1e-12, atol=1e-12)


def test_scaling_down_projection_by_two_doubles_output_exactly():
    cfg, lg, x, w13, w2 = _tiny(T=20, E=5, k=2)
    a = o.layer_forward(cfg, lg, x, w13, w2)["out"]
    b = o.layer_forward(cfg, lg, x, w13, 2.0 * w2)["out"]
    assert (b == 2.0 * a).all()


def test_identity_experts_recover_tokens():
    """If every expert returned its input row, the weighted combine of a
    token's k rows (weights summing to 1) gives back the token: pins that
    combine reads assign_to_row as the inverse of the packing."""
    cfg, lg, x, w13, w2 = _tiny(T=40, E=6, k=3, n_hot_split=2, split_ways=2)
    ids, w, _ = o.route(cfg, lg)
    p = o.plan(cfg, ids)
    x_perm = x[p["row_to_token"]]
    out = o.combine(x_perm, p["assign_to_row"], w)
    np.testing.assert_allclose(out, x, rtol=1e-13, atol=1e-14)
    # and with distinct per-slot weights the pairing of slot and row matters
    y = x_perm * (1.0 + p["row_to_assign"][:, None] % cfg.k)
    out2 = o.combine(y, p["assign_to_row"], w)
    np.testing.assert_allclose(out2, x * (w * (1.0 + np.arange(cfg.k))).sum(1, keepdims=True), rtol=1e-13)


def test_replica_segments_do_not_change_the_output():
    """Replication changes where an expert runs, not which experts or
    weights a token gets (Zepp section 4.1): splitting hot experts by token
    parity gives the same output, bit for bit, in the oracle."""
    cfg, lg, x, w13, w2 = _tiny(T=45, E=6, k=3, n_hot_split=2, split_ways=2)
    a = o.layer_forward(cfg, lg, x, w13, w2)
    b = o.layer_forward(cfg.replace(n_hot_split=0, split_ways=1), lg, x, w13, w2)
    assert len(a["seg_expert"]) == 8 and len(b["seg_expert"]) == 6
    assert (a["out"] == b["out"]).all()


def test_shared_expert_is_added_with_weight_one():
    """Shared experts process every token, independent of routing ("MoE
    architecture recap")."""
    cfg, lg, x, w13, w2 = _tiny(T=12, E=4, k=2)
    rng = np.random.default_rng(3)
    sw13 = rng.standard_normal((2 * 8, 16)) * 0.3
    sw2 = rng.standard_normal((16, 8)) * 0.3
    a = o.layer_forward(cfg, lg, x, w13, w2)
    b = o.layer_forward(cfg, lg, x, w13, w2, sw13, sw2)
    np.testing.assert_allclose(b["out"] - a["out"], _dense(x, sw13, sw2), rtol=1e-11, atol=1e-12)


def test_token_outputs_match_whole_layer():
    """The sampled per-token form equals the permuted whole-layer form."""
    cfg, lg, x, w13, w2 = _tiny(T=30, E=6, k=3, n_hot_split=1, split_ways=2)
    r = o.layer_forward(cfg, lg, x, w13, w2)
    toks = [0, 7, 29]
    out = o.token_outputs(toks, x[toks], r["ids"][toks], r["w"][toks], lambda e: (w13[e], w2[e]))
    np.testing.assert_allclose(out, r["out"][toks], rtol=1e-12, atol=1e-13)
