"""Pins for the oracle's acceptance and compaction.

Greedy: aiunderstanding.org "Medusa Decoding Heads" ("Deep Dive", the longest
prefix matching what the model would have produced) and inferensys.com
"Medusa Heads" (stop at the first rejection): the token-by-token argmax
replay must agree with the parallel flag formulation, and planted paths must
come back.  Typical: aicassindra.com "Medusa deep dive", "Typical acceptance,
not exact rejection sampling": closed-form limits of min(eps, delta e^-H).
"""

import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import (tree_plan, accept_greedy_walk, accept_greedy_parallel,
                    accept_typical, typical_local, kv_compact, full_tree_node_count)


def _tree_tokens(plan, V, rng):
    """Distinct tokens among siblings, as a top-k shortlist would give."""
    tokens = np.zeros(plan.T, dtype=np.int64)
    tokens[0] = rng.integers(V)
    for p in range(plan.T):
        kids = [c for c in range(1, plan.T) if plan.parent[c] == p]
        if kids:
            tokens[kids] = rng.choice(V, size=len(kids), replace=False)
    return tokens


@settings(max_examples=80, deadline=None)
@given(k=st.lists(st.integers(1, 4), min_size=1, max_size=4), frac=st.floats(0, 1),
       seed=st.integers(0, 10 ** 6), plant=st.floats(0, 1))
def test_greedy_walk_equals_parallel(k, frac, seed, plant):
    N = int(round(frac * full_tree_node_count(k)))
    plan = tree_plan(k, N)
    rng = np.random.default_rng(seed)
    V = 12
    tokens = _tree_tokens(plan, V, rng)
    logits = rng.standard_normal((plan.T, V))
    # plant matches along random edges so that long paths occur
    for c in range(1, plan.T):
        if rng.random() < plant:
            logits[plan.parent[c], tokens[c]] = logits[plan.parent[c]].max() + 1.0
    K = len(k)
    a = accept_greedy_walk(logits, tokens, plan.parent, K)
    b = accept_greedy_parallel(logits, tokens, plan.parent, plan.depth, K)
    assert a[0] == b[0] and list(a[1]) == list(b[1]) and list(a[2]) == list(b[2]) and a[3] == b[3]


def test_greedy_planted_path_comes_back():
    plan = tree_plan((10,) * 4, 64)
    rng = np.random.default_rng(1)
    V = 64
    for target in [5, 20, 40, plan.T - 1]:
        tokens = _tree_tokens(plan, V, rng)
        logits = rng.standard_normal((plan.T, V))
        chain = []
        j = target
        while j >= 0:
            chain.append(j)
            j = plan.parent[j]
        chain.reverse()
        for p, c in zip(chain[:-1], chain[1:]):
            logits[p, tokens[c]] = logits[p].max() + 1.0
        # make sure the chain ends: nothing below the target matches
        amax_t = int(np.argmax(logits[target]))
        kids = [c for c in range(plan.T) if plan.parent[c] == target]
        for c in kids:
            if tokens[c] == amax_t:
                logits[target, amax_t] -= 10.0
        # and no deeper sibling path beats it: remove accidental matches elsewhere
        L, path, acc, bonus = accept_greedy_walk(logits, tokens, plan.parent, 4)
        assert L == plan.depth[target]
        assert list(path[: L + 1]) == chain
        assert list(acc[: L + 1]) == [int(tokens[c]) for c in chain]
        assert bonus == int(np.argmax(logits[target]))
        assert all(x == -1 for x in path[L + 1:])


def test_greedy_nothing_matches():
    plan = tree_plan((2, 2), None)
    logits = np.zeros((plan.T, 10))
    logits[:, 9] = 1.0                                  # argmax 9 everywhere
    tokens = np.array([0, 1, 2, 3, 4, 5, 6])
    L, path, acc, bonus = accept_greedy_walk(logits, tokens, plan.parent, 2)
    assert (L, list(path), list(acc), bonus) == (0, [0, -1, -1], [0, -1, -1], 9)


def _entropy(q):
    q = np.asarray(q)
    q = q[q > 0]
    return float(-(q * np.log(q)).sum())


def test_typical_uniform_accepts_everything():
    # uniform q: H = ln V, threshold = min(eps, delta / V) = delta / V < 1/V = q
    V = 50
    ok, q, thr, H = typical_local(np.zeros(V), 3, 0.7, 0.3, 0.09)
    assert ok and abs(H - math.log(V)) < 1e-12 and abs(thr - 0.09 / V) < 1e-15
    plan = tree_plan((3, 3, 2), None)
    rng = np.random.default_rng(2)
    tokens = _tree_tokens(plan, V, rng)
    L, path, acc, bonus, _ = accept_typical(np.zeros((plan.T, V)), tokens, plan.parent,
                                            plan.depth, 3, 0.7, 0.3, 0.09, 1, 0, 0)
    assert L == 3
    deepest = min(i for i in range(plan.T) if plan.depth[i] == 3)
    assert path[-1] == deepest


def test_typical_peaked_tracks_greedy():
    # a peaked model accepts only its argmax: typical == greedy
    plan = tree_plan((4, 4, 4), 30)
    rng = np.random.default_rng(3)
    V = 40
    for _ in range(20):
        tokens = _tree_tokens(plan, V, rng)
        logits = rng.standard_normal((plan.T, V))
        for c in range(1, plan.T):
            if rng.random() < 0.6:
                logits[plan.parent[c], tokens[c]] = logits[plan.parent[c]].max() + 1.0
        logits *= 40.0
        g = accept_greedy_parallel(logits, tokens, plan.parent, plan.depth, 3)
        t = accept_typical(logits, tokens, plan.parent, plan.depth, 3, 0.7, 0.3, 0.09, 5, 0, 0)
        assert g[0] == t[0] and list(g[1]) == list(t[1])


def test_typical_one_hot_limit_threshold_is_delta():
    row = np.array([0.0, 500.0, 0.0, 0.0])
    ok, q, thr, H = typical_local(row, 1, 1.0, 0.3, 0.09)
    assert ok and H < 1e-100 and abs(thr - 0.09) < 1e-15
    ok, q, thr, H = typical_local(row, 0, 1.0, 0.3, 0.09)
    assert not ok


def test_typical_eps_branch_switches_at_log_delta_over_eps():
    # with eps < delta the threshold is eps while H < ln(delta/eps)
    eps, delta = 0.02, 0.5
    Hs = math.log(delta / eps)
    # two-level distribution on V tokens with tunable entropy
    V = 64
    for gap in (8.0, 4.0, 2.0, 1.0, 0.5, 0.0):
        row = np.zeros(V)
        row[0] = gap
        q = np.exp(row - row.max())
        q /= q.sum()
        H = _entropy(q)
        ok, qt, thr, Hgot = typical_local(row, 5, 1.0, eps, delta)
        assert abs(Hgot - H) < 1e-12
        want = eps if H < Hs else delta * math.exp(-H)
        assert abs(thr - want) < 1e-15
        assert ok == (q[5] > want)


def test_typical_temperature_is_applied():
    row = np.array([0.0, 1.0, 2.0])
    _, q1, _, _ = typical_local(row, 2, 1.0, 0.3, 0.09)
    _, q2, _, _ = typical_local(row, 2, 0.5, 0.3, 0.09)
    assert abs(q1 - math.exp(2) / (1 + math.e + math.exp(2))) < 1e-15
    assert abs(q2 - math.exp(4) / (1 + math.exp(2) + math.exp(4))) < 1e-15


# ---------------------------------------------------------------- compaction
def test_compact_chain_path_is_noop():
    rng = np.random.default_rng(4)
    Kc, Vc = rng.standard_normal((2, 20, 4)), rng.standard_normal((2, 20, 4))
    Kn, Vn, n = kv_compact(Kc, Vc, 10, [0, 1, 2, -1], 2)
    assert np.array_equal(Kn, Kc) and np.array_equal(Vn, Vc) and n == 13


def test_compact_overlapping_moves_read_before_write():
    rng = np.random.default_rng(5)
    Kc, Vc = rng.standard_normal((3, 30, 4)), rng.standard_normal((3, 30, 4))
    P = 8
    Kn, Vn, n = kv_compact(Kc, Vc, P, [0, 2, 5, -1], 2)
    assert n == P + 3
    assert np.array_equal(Kn[:, :P], Kc[:, :P])
    assert np.array_equal(Kn[:, P + 1], Kc[:, P + 2])
    assert np.array_equal(Kn[:, P + 2], Kc[:, P + 5])   # the old slot, not the moved one
    assert np.array_equal(Vn[:, P + 2], Vc[:, P + 5])
    assert np.array_equal(Kn[:, P + 3:], Kc[:, P + 3:])


def test_compact_nothing_accepted():
    rng = np.random.default_rng(6)
    Kc, Vc = rng.standard_normal((1, 12, 2)), rng.standard_normal((1, 12, 2))
    Kn, Vn, n = kv_compact(Kc, Vc, 4, [0, -1, -1], 0)
    assert n == 5 and np.array_equal(Kn, Kc)
