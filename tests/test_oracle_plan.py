"""Pins for the oracle's planner (blog, "How each query picks its own depth": reverse
water-filling over channel importance, 0..4 planes per channel, the budget spent
exactly; equal keys go to the lower channel index).

Independent checks: the sorted-prefix formulation (numpy lexsort), exhaustive search
for the optimum on tiny d (exact rationals), closed-form cases and the exchange
(KKT) condition of water-filling.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def _w(q, var):
    q64 = q.astype(np.float64)
    return (q64 * q64).sum(axis=0) * var.astype(np.float64)


def _plan_from_w(var, B, G=1):
    """Feed w through the oracle with q = 1 (G=1), so w_c = var_c."""
    d = var.shape[0]
    q = np.ones((G, d), np.float32)
    return oracle.plan(q, var.astype(np.float32), B)


def test_budget_edges():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    var = rng.uniform(0.01, 10, 128).astype(np.float32)
    assert (oracle.plan(q, var, 0) == 0).all()
    assert (oracle.plan(q, var, 512) == 4).all()
    with pytest.raises(ValueError):
        oracle.plan(q, var, 513)
    with pytest.raises(ValueError):
        oracle.plan(q, var, -1)


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), B=st.integers(0, 512), G=st.integers(1, 8))
def test_plan_sums_to_budget_and_is_bounded(seed, B, G):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, 128)).astype(np.float32)
    var = (10 ** rng.uniform(-2, 2, 128)).astype(np.float32)
    depth = oracle.plan(q, var, B)
    assert int(depth.sum()) == B
    assert depth.max() <= 4


def test_equal_importance_closed_forms():
    var = np.ones(128, np.float32)
    d136 = _plan_from_w(var, 136)
    assert (d136[:8] == 2).all() and (d136[8:] == 1).all()
    d92 = _plan_from_w(var, 92)
    assert (d92[:92] == 1).all() and (d92[92:] == 0).all()


@pytest.mark.parametrize("B,expect", [(3, (2, 1, 0)), (5, (3, 2, 0)), (8, (4, 4, 0)),
                                      (9, (4, 4, 1))])
def test_small_weights_closed_forms(B, expect):
    var = np.zeros(6, np.float32)
    var[0], var[1] = 4.0, 1.0
    depth = _plan_from_w(var, B)
    assert tuple(int(t) for t in depth[:3]) == expect
    assert int(depth.sum()) == B


def _sorted_prefix(w, B):
    """Items (c, t) with key w_c * 4^-t, ordered by key desc, then c, then t."""
    d = w.shape[0]
    c = np.repeat(np.arange(d), 4)
    t = np.tile(np.arange(4), d)
    key = np.ldexp(w[c], -2 * t)
    order = np.lexsort((t, c, -key))
    depth = np.zeros(d, np.int64)
    for i in order[:B]:
        depth[c[i]] += 1
    return depth


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), B=st.integers(0, 512), ties=st.booleans())
def test_greedy_equals_sorted_prefix(seed, B, ties):
    rng = np.random.default_rng(seed)
    G = int(rng.integers(1, 5))
    q = rng.standard_normal((G, 128)).astype(np.float32)
    var = (10 ** rng.uniform(-2, 2, 128)).astype(np.float32)
    if ties:   # heavy ties: few distinct importances, some exactly 4x apart
        q = np.ones((1, 128), np.float32)
        var = rng.choice(np.array([0, 1, 4, 16, 2], np.float32), 128)
    depth = oracle.plan(q, var, B)
    assert (depth == _sorted_prefix(_w(q, var), B)).all()


def _frac(x):
    return Fraction(float(x))


@pytest.mark.parametrize("d", [1, 2, 3, 4, 5])
def test_greedy_is_optimal_by_exhaustive_search(d):
    rng = np.random.default_rng(100 + d)
    for trial in range(20):
        var = rng.choice(np.array([0, 0.5, 1, 2, 4, 3, 16], np.float32), d) \
            if trial % 2 else (10 ** rng.uniform(-2, 2, d)).astype(np.float32)
        w = [_frac(v) for v in var]
        for B in range(0, 4 * d + 1):
            depth = _plan_from_w(var, B)
            got = sum(w[c] / 4 ** int(depth[c]) for c in range(d))
            best = min(sum(w[c] / 4 ** t[c] for c in range(d))
                       for t in itertools.product(range(5), repeat=d) if sum(t) == B)
            assert got == best, (d, trial, B)


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), B=st.integers(1, 511))
def test_exchange_condition(seed, B):
    """No plane can move from channel b to channel a and lower the distortion:
    if t_a < 4 and t_b > 0 then w_a 4^-t_a <= w_b 4^-(t_b - 1)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    var = (10 ** rng.uniform(-3, 3, 128)).astype(np.float32)
    depth = oracle.plan(q, var, B).astype(int)
    w = [_frac(x) for x in _w(q, var)]
    gain_next = [w[c] / 4 ** depth[c] if depth[c] < 4 else None for c in range(128)]
    gain_last = [w[c] / 4 ** (depth[c] - 1) if depth[c] > 0 else None for c in range(128)]
    lo = min(g for g in gain_last if g is not None)
    hi = max(g for g in gain_next if g is not None)
    assert hi <= lo


def test_importance_sums_queries_of_one_kv_head():
    q = np.array([[1.0, 2.0], [3.0, -1.0]], np.float32)
    var = np.array([0.5, 2.0], np.float32)
    assert oracle.importance(q, var, 0) == (1 + 9) * 0.5
    assert oracle.importance(q, var, 1) == (4 + 1) * 2.0


@pytest.mark.parametrize("F", [0, 1, 34, 127, 128])
def test_fixed_plan_matches_stable_argsort(F):
    rng = np.random.default_rng(F)
    var = rng.choice(np.array([0, 0.5, 1, 2, 3], np.float32), 128)   # many ties
    depth = oracle.plan_fixed(var, F)
    order = np.argsort(-var.astype(np.float64), kind="stable")    # ties: lower index
    ref = np.zeros(128, np.uint8)
    ref[order[:F]] = 4
    assert (depth == ref).all()
    assert int(depth.sum()) == 4 * F
