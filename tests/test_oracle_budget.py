"""Pins of the tree-budget oracle (oracle/budget.py) against what the pages and
the mathematics fix, independently of the planner's own formula:

  * optimality: the planned N-tree has the largest expected tokens among every
    ancestor-closed set of N candidates (brute force over all subsets);
  * expected tokens: equal to the exact expectation of 1 + L over every
    outcome of independent per-head true ranks (aicassindra.com "Medusa deep
    dive", "What it costs on a CPU-bound SLM": tokens confirmed per pass;
    "The conditional-independence gap": heads see only the hidden state);
  * the fixed rule decay^d / (rank + 1) is the special case of the rates
    planner wherever its exact ranking has a strict cut-off;
  * the tally on a hand-derived example, and the tally's rate estimate
    recovering known rates in a seeded simulation of greedy acceptance.
"""

from fractions import Fraction
from itertools import combinations, product

import numpy as np
import pytest

from oracle import accept_tally, expected_tokens, plan_from_tables, tree_plan, tree_plan_rates
from oracle.tree import tuple_score

def _all_tuples(k):
    out = []
    for D in range(1, len(k) + 1):
        out.extend(product(*[range(s) for s in k[:D]]))
    return out

def _rand_q(k, seed, rows_sum_le_one=False):
    rng = np.random.default_rng(seed)
    q = np.zeros((len(k), 16))
    for d, s in enumerate(k):
        v = rng.random(s)
        if rows_sum_le_one:
            v = v / v.sum() * rng.uniform(0.3, 0.95)
        q[d, :s] = v
    return q

@pytest.mark.parametrize("k,seed", [((2, 2, 2), 1), ((3, 2, 1), 2), ((1, 3, 2), 3)])
def test_planned_tree_is_optimal_among_ancestor_closed_sets(k, seed):
    q = _rand_q(k, seed)
    tuples = _all_tuples(k)
    best = {}
    for n in range(len(tuples) + 1):
        for sub in combinations(tuples, n):
            s = set(sub)
            if any(t[:-1] and t[:-1] not in s for t in sub):
                continue
            val = 1.0 + sum(float(np.prod([q[d][r] for d, r in enumerate(t)])) for t in sub)
            best[n] = max(best.get(n, 0.0), val)
    for n in range(len(tuples) + 1):
        _, e = tree_plan_rates(k, n, q)
        assert abs(e - best[n]) < 1e-12, (n, e, best[n])

def _exact_expected_tokens(plan, k, qf):
    """1 + E[L] by enumerating each depth's true rank (or none) exactly."""
    nodes = set(plan.tuples)
    K = len(k)
    total = Fraction(0)
    choices = [list(range(s)) + [None] for s in k]
    for outcome in product(*choices):
        p = Fraction(1)
        for d, r in enumerate(outcome):
            p *= (1 - sum(qf[d])) if r is None else qf[d][r]
        if p == 0:
            continue
        L = 0
        for D in range(1, K + 1):
            if outcome[D - 1] is None or tuple(outcome[:D]) not in nodes:
                break
            L = D
        total += p * (1 + L)
    return total

@pytest.mark.parametrize("N", [0, 1, 3, 7, 12, 20])
def test_expected_tokens_equals_exact_expectation(N):
    k = (3, 3, 2)
    rng = np.random.default_rng(7)
    qf = []
    for s in k:
        w = [Fraction(int(x), 40) for x in rng.integers(1, 12, size=s)]
        qf.append(w)                       # each row sums to at most 33/40
    q = np.zeros((3, 16))
    for d in range(3):
        q[d, : k[d]] = [float(x) for x in qf[d]]
    plan, e = tree_plan_rates(k, N, q)
    want = _exact_expected_tokens(plan, k, qf)
    assert abs(e - float(want)) < 1e-12
    assert abs(expected_tokens(plan, q) - e) == 0.0

def test_fixed_rule_is_the_rates_planner_at_strict_cutoffs():
    k = (10, 10, 10, 10)
    decay = Fraction(4, 5)
    q = np.zeros((4, 16))
    for d in range(4):
        for r in range(10):
            q[d, r] = float(decay ** (d + 1) / (r + 1))
    scores = sorted((tuple_score(t, decay) for t in _all_tuples(k)), reverse=True)
    # cut-offs with a strict gap (scores are ratios of small integers and tie
    # often; inside a tie the float product order may differ from the exact one)
    strict = [N for N in range(1, 256)
              if float(scores[N - 1]) / float(scores[N]) > 1 + 1e-12]
    assert len(strict) >= 20
    for N in strict[:: max(1, len(strict) // 10)]:
        fixed = tree_plan(k, N, decay)
        rates, _ = tree_plan_rates(k, N, q)
        assert fixed.tuples == rates.tuples, N

def test_tally_hand_example():
    # full tree of k = (2, 2): nodes (), (0), (1), (0,0), (0,1), (1,0), (1,1)
    plan, _ = tree_plan_rates((2, 2), None, np.ones((2, 16)))
    assert plan.tuples == [(), (0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)]
    L = np.array([2, 0, 1])
    path = np.array([[0, 1, 3], [0, -1, -1], [0, 2, -1]])
    acc, off = accept_tally(plan, 2, L, path)
    assert off[0, :2].tolist() == [3, 3] and acc[0, :2].tolist() == [1, 1]
    assert off[1, :2].tolist() == [2, 2] and acc[1, :2].tolist() == [1, 0]
    assert acc[:, 2:].sum() == 0 and off[:, 2:].sum() == 0

def test_tally_estimate_recovers_rates_in_simulation():
    k = (3, 3, 3)
    K = len(k)
    q = _rand_q(k, 11, rows_sum_le_one=True)
    plan, _ = tree_plan_rates(k, 20, q)
    index = {t: i for i, t in enumerate(plan.tuples)}
    rng = np.random.default_rng(12)
    steps = 20000
    L = np.zeros(steps, dtype=np.int64)
    path = np.full((steps, K + 1), -1, dtype=np.int64)
    for s in range(steps):
        path[s, 0] = 0
        t = ()
        for d in range(K):
            u = rng.random()
            cum = np.cumsum(q[d, : k[d]])
            r = int(np.searchsorted(cum, u, side="right"))
            if r >= k[d] or t + (r,) not in index:
                break
            t = t + (r,)
            path[s, d + 1] = index[t]
            L[s] = d + 1
    acc, off = accept_tally(plan, K, L, path)
    for d in range(K):
        for r in range(k[d]):
            if off[d, r] < 200:
                continue
            est = acc[d, r] / off[d, r]
            sd = np.sqrt(q[d, r] * (1 - q[d, r]) / off[d, r])
            assert abs(est - q[d, r]) < 5 * sd + 1e-9, (d, r, est, q[d, r])

def test_plan_from_tables_round_trip_and_rejections():
    q = _rand_q((4, 3, 2), 5)
    plan, _ = tree_plan_rates((4, 3, 2), 13, q)
    ranks = [-1] + [t[-1] for t in plan.tuples[1:]]
    back = plan_from_tables((4, 3, 2), plan.parent, ranks)
    assert back.tuples == plan.tuples
    assert (back.anc == plan.anc).all()
    with pytest.raises(ValueError):
        plan_from_tables((2, 2), [-1, 0, 3, 1], [-1, 0, 1, 0])       # parent after node
    with pytest.raises(ValueError):
        plan_from_tables((2, 2), [-1, 0, 0], [-1, 0, 2])             # rank >= k
    with pytest.raises(ValueError):
        plan_from_tables((2, 2), [-1, 0, 0], [-1, 1, 1])             # duplicate child
    with pytest.raises(ValueError):
        plan_from_tables((2, 2), [-1, 0, 1, 0], [-1, 0, 0, 1])       # depth decreases
    with pytest.raises(ValueError):
        plan_from_tables((2,), [-1, 0, 1], [-1, 0, 0])               # deeper than K
