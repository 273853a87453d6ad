"""Pins for the oracle's tree planner, mask and gather.

Each check compares the oracle with something it does not compute itself:
the node and path counts printed on zackli.ai "Speculative Decoding Deep Dive
II" (section "Medusa"), hand-derived plans in tests/golden/, and the
prefix relation of rank tuples as an independent definition of Anc(i).
"""

import os
import re
from itertools import product

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import tree_plan, tree_gather, full_tree_node_count, full_path_count

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _tuples(s):
    out = []
    for tok in s.split():
        inner = tok.strip("()")
        out.append(tuple(int(x) for x in inner.split(",")) if inner else ())
    return out


def test_full_tree_counts_closed_form():
    # tree nodes = s1 + s1 s2 + s1 s2 s3 + ...; full paths = s1 s2 s3 ...
    for k, nodes, paths in [((2, 2, 1), 2 + 4 + 4, 4), ((3,), 3, 3),
                            ((2, 3, 4), 2 + 6 + 24, 24), ((1, 1, 1, 1), 4, 1),
                            ((10, 10, 10, 10), 11110, 10000)]:
        assert full_tree_node_count(k) == nodes
        assert full_path_count(k) == paths
        if nodes <= 200:
            plan = tree_plan(k)
            assert plan.T == nodes + 1
            assert int((plan.depth == len(k)).sum()) == paths


def test_tiny_workload_is_full_tree_of_ten():
    plan = tree_plan((2, 2, 1))
    assert plan.T == 11
    assert list(np.bincount(plan.depth)) == [1, 2, 4, 4]


def test_hand_worked_sparse_plans():
    with open(os.path.join(GOLD, "tree_k3x2.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    assert rows
    for ln in rows:
        n, nodes, parent, depth = [p.strip() for p in ln.split("|")]
        plan = tree_plan((3, 2), int(n))
        assert plan.tuples == _tuples(nodes)
        assert list(plan.parent) == [int(x) for x in parent.split()]
        assert list(plan.depth) == [int(x) for x in depth.split()]


def _golden_kv(name):
    d = {}
    with open(os.path.join(GOLD, name)) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                key, rest = ln.split(None, 1)
                d[key] = rest.strip()
    return d


@pytest.mark.parametrize("fname,k,N", [("tree_k10x4_n64.txt", (10,) * 4, 64),
                                       ("tree_k10x5_n128.txt", (10,) * 5, 128)])
def test_large_sparse_plans_match_hand_derivation(fname, k, N):
    g = _golden_kv(fname)
    plan = tree_plan(k, N)
    hist = np.bincount(plan.depth, minlength=len(k) + 1)[1:]
    assert list(hist) == [int(x) for x in g["hist"].split()]
    kept = set(plan.tuples)
    for t in _tuples(g["tie_in"]):
        assert t in kept
    for t in _tuples(g["tie_out"]):
        assert t not in kept
    for key in ("depth4", "depth5"):
        if key in g:
            D = int(key[-1])
            assert sorted(t for t in plan.tuples if len(t) == D) == sorted(_tuples(g[key]))


def _check_plan_invariants(plan):
    T = plan.T
    assert plan.tuples[0] == () and plan.parent[0] == -1 and plan.depth[0] == 0
    for i in range(1, T):
        p = plan.parent[i]
        assert 0 <= p < i                                   # parent before child
        assert plan.tuples[p] == plan.tuples[i][:-1]        # ancestor-closed
        assert plan.depth[i] == plan.depth[p] + 1
    # Anc(i) from the prefix relation of rank tuples (independent of parent walk)
    for i in range(T):
        for j in range(T):
            ti, tj = plan.tuples[i], plan.tuples[j]
            assert plan.anc[i, j] == (ti[: len(tj)] == tj)


@settings(max_examples=60, deadline=None)
@given(k=st.lists(st.integers(1, 4), min_size=1, max_size=4), frac=st.floats(0.0, 1.0))
def test_plan_invariants_random(k, frac):
    total = full_tree_node_count(k)
    N = int(round(frac * total))
    plan = tree_plan(k, N)
    assert plan.T == N + 1
    _check_plan_invariants(plan)


def test_plan_invariants_workload_trees():
    for k, N in [((2, 2, 1), None), ((10,) * 4, 64), ((10,) * 5, 128)]:
        _check_plan_invariants(tree_plan(k, N))


def test_sparse_tree_prefers_confident_early_heads():
    # every kept candidate outranks every dropped one in the ranking rule: check
    # with floats in log space, a route independent of the Fraction sort
    k, N = (4, 3, 2), 9
    plan = tree_plan(k, N)
    kept = set(plan.tuples[1:])

    def logscore(t):
        return sum(d * np.log(0.8) - np.log(r + 1) for d, r in enumerate(t, 1))

    every = [t for D in range(1, 4) for t in product(*[range(s) for s in k[:D]])]
    lo = min(logscore(t) for t in kept)
    hi = max(logscore(t) for t in every if t not in kept)
    assert lo >= hi - 1e-12


def test_gather_hand_example():
    plan = tree_plan((3, 2), 5)
    idx = np.array([[7, 3, 9], [4, 8, -1]])
    tokens, pos = tree_gather(plan, 11, idx, 100)
    assert list(tokens) == [11, 7, 3, 9, 4, 8]
    assert list(pos) == [100, 101, 101, 101, 102, 102]


def test_too_many_candidates_rejected():
    with pytest.raises(ValueError):
        tree_plan((2, 2), 7)
