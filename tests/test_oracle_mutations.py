"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, by replacing one of
its functions for the duration of the check) and runs every pin of
test_oracle_pins; at least one pin must fail.  A pin suite that still passed
would not pin that part of the oracle.
"""
import contextlib
import inspect

import numpy as np
import pytest

from oracle import moe_oracle as o
from tests import test_oracle_pins as pins


@contextlib.contextmanager
def planted(name, fn):
    orig = getattr(o, name)
    setattr(o, name, fn)
    try:
        yield
    finally:
        setattr(o, name, orig)


def _pin_calls():
    """Every pin as a zero-argument callable (parametrised pins expanded)."""
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argnames = [a.strip() for a in params[0].args[0].split(",")]
            for vals in params[0].args[1]:
                vals = vals if isinstance(vals, tuple) else (vals,)
                calls.append((name, lambda fn=fn, kw=dict(zip(argnames, vals)): fn(**kw)))
        else:
            calls.append((name, fn))
    return calls


def _failing_pins():
    failed = []
    for name, call in _pin_calls():
        try:
            call()
        except Exception:  # an assertion, or a shape error from a transposed operand
            failed.append(name)
    return failed


# ---------------------------------------------------------------- mistakes
orig_route_flat = o.route_flat
orig_route_grouped = o.route_grouped
orig_swiglu = o.swiglu
orig_combine = o.combine
orig_permutation = o.permutation
orig_hot = o.hot_experts
orig_gs = o.group_scores_f32


def ascending_route(logits, k, renormalize=True):
    ids, w = orig_route_flat(-np.asarray(logits, dtype=np.float32), k, renormalize)
    return ids, w


def never_renormalised(logits, k, renormalize=True):
    return orig_route_flat(logits, k, False)


def reversed_weights(logits, k, renormalize=True):
    ids, w = orig_route_flat(logits, k, renormalize)
    return ids, w[:, ::-1].copy()


def max_member_group_score(logits, n_group, topn):
    return orig_gs(logits, n_group, 1)


def worst_groups(logits, k, n_group, topk_group, topn=2, renormalize=True):
    return orig_route_grouped(-np.asarray(logits, dtype=np.float32), k, n_group, topk_group, topn,
                              renormalize)


def silu_on_up(x_rows, w13_e, w2_e):
    I = w13_e.shape[0] // 2
    return orig_swiglu(x_rows, np.concatenate([w13_e[I:], w13_e[:I]]), w2_e)


def down_transposed(x_rows, w13_e, w2_e):
    return orig_swiglu(x_rows, w13_e, w2_e.T)


def unweighted_combine(y_perm, assign_to_row, w, shared_y=None):
    return orig_combine(y_perm, assign_to_row, np.ones_like(w), shared_y)


def wrong_inverse(seg_of_a, S, k):
    so, r2a, a2r, r2t = orig_permutation(seg_of_a, S, k)
    return so, r2a, r2a, r2t   # row_to_assign where assign_to_row belongs


def unstable_rows(seg_of_a, S, k):
    so, r2a, a2r, r2t = orig_permutation(seg_of_a, S, k)
    r2a = r2a.copy()
    for s in range(S):
        r2a[so[s]:so[s + 1]] = r2a[so[s]:so[s + 1]][::-1]
    a2r = np.empty_like(r2a)
    a2r[r2a] = np.arange(r2a.size)
    return so, r2a, a2r.astype(np.int32), (r2a // k).astype(np.int32)


def inverted_balancedness(loads):
    loads = np.asarray(loads, dtype=np.float64)
    return np.float32(loads.max() / loads.mean())


def active_only_balancedness(loads):
    loads = np.asarray(loads, dtype=np.float64)
    return np.float32(loads[loads > 0].mean() / loads.max())


def coldest_are_hot(counts, n_hot):
    return sorted(range(len(counts)), key=lambda e: (int(counts[e]), e))[:n_hot]


orig_soa = o.segment_of_assignments
orig_replica_loads = o.replica_loads


def no_reservation(d, ways, c_permille):
    """Fills each replica to its upper bound without keeping back the later
    replicas' lower bounds."""
    q = o.Fraction(d, ways)
    ub = o.math.ceil(q * (1 + o.Fraction(c_permille, 1000)))
    loads, left = [], d
    for _ in range(ways):
        n = min(ub, left)
        loads.append(n)
        left -= n
    return loads


def floor_upper_bound(d, ways, c_permille):
    q = o.Fraction(d, ways)
    C = o.Fraction(c_permille, 1000)
    lb, ub = max(0, o.math.floor(q * (1 - C))), o.math.floor(q * (1 + C))
    loads, left = [], d
    for p in range(ways):
        n = left if p == ways - 1 else min(ub, left - (ways - 1 - p) * lb)
        loads.append(n)
        left -= n
    return loads


def last_replica_first(d, ways, c_permille):
    return orig_replica_loads(d, ways, c_permille)[::-1]


def parity_for_bounded(ids, seg_expert, seg_replica, ways, loads=None):
    return orig_soa(ids, seg_expert, seg_replica, ways, None)


orig_capacity_plan = o.capacity_plan


def capacity_rounded_down(A, E, factor_permille):
    return A * factor_permille // (1000 * E)


def keeps_the_latest(ids, E, cap):
    """Drops the earliest assignments of a full expert instead of the latest."""
    rev = ids.ravel()[::-1].reshape(ids.shape[0] * ids.shape[1], 1)
    p = orig_capacity_plan(rev, E, cap)
    k = ids.shape[1]
    a2r = p["assign_to_row"][::-1].copy()
    r2a = np.full(E * cap, -1)
    r2a[a2r[a2r >= 0]] = np.nonzero(a2r >= 0)[0]
    p.update(assign_to_row=a2r, row_to_assign=r2a, row_to_token=np.where(r2a >= 0, r2a // k, -1))
    return p


def never_drops(ids, E, cap):
    return orig_capacity_plan(ids, E, max(cap, int(np.bincount(ids.ravel(), minlength=E).max())))


def dropped_rows_wrap_around(y_perm, assign_to_row, w, shared_y=None):
    T, k = w.shape
    out = np.zeros((T, y_perm.shape[1]))
    for a in range(T * k):
        out[a // k] += w[a // k, a % k] * y_perm[assign_to_row[a]]   # row -1: the last row
    return out if shared_y is None else out + shared_y


MISTAKES = [
    ("route_flat", ascending_route),
    ("route_flat", never_renormalised),
    ("route_flat", reversed_weights),
    ("group_scores_f32", max_member_group_score),
    ("route_grouped", worst_groups),
    ("swiglu", silu_on_up),
    ("swiglu", down_transposed),
    ("combine", unweighted_combine),
    ("permutation", wrong_inverse),
    ("permutation", unstable_rows),
    ("balancedness", inverted_balancedness),
    ("balancedness", active_only_balancedness),
    ("hot_experts", coldest_are_hot),
    ("replica_loads", no_reservation),
    ("replica_loads", floor_upper_bound),
    ("replica_loads", last_replica_first),
    ("segment_of_assignments", parity_for_bounded),
    ("capacity", capacity_rounded_down),
    ("capacity_plan", keeps_the_latest),
    ("capacity_plan", never_drops),
    ("combine", dropped_rows_wrap_around),
]


def test_pins_pass_on_the_unmodified_oracle():
    assert _failing_pins() == []


@pytest.mark.parametrize("name,fn", MISTAKES, ids=[f.__name__ for _, f in MISTAKES])
def test_planted_mistake_is_caught(name, fn):
    with planted(name, fn):
        failed = _failing_pins()
    assert failed, f"no pin catches {fn.__name__} in {name}"
