"""Tree budget from measured acceptance rates (oracle).

Test infrastructure only.

Pages:
  * aicassindra.com "Medusa deep dive", "From top-k heads to a sparse candidate
    tree": the sparse tree is chosen ahead of time, giving more branches to
    confident, early heads, and its shape is a tuned budget that trades more
    candidates (higher acceptance) against a heavier verification pass.
  * same page, "What it costs on a CPU-bound SLM": the expected acceptance
    length (tokens confirmed per pass) multiplies throughput; K and the tree
    size are tuned against the decay of per-head accuracy with offset.
  * same page, "The conditional-independence gap": every head conditions on the
    same hidden state and nothing else.

Readings (the pages give the objective, not the procedure):
  * q[d][r] is the rate at which the rank-r candidate of head d+1 is accepted
    given that its parent was: the fraction of steps in which that node was
    offered (its parent lay on the accepted path) and accepted.
  * Heads are taken as independent given the hidden state (the independence
    gap), so a node's path is accepted with probability
    prod_d q[d][r_d], and at most one node per depth lies on the accepted
    path.  Expected tokens per step = 1 (the base model's own next token) +
    the sum of those products over the tree's candidates.
  * The N-candidate tree with the most expected tokens keeps the N tuples of
    largest product (q <= 1 makes a child score no higher than its parent, so
    the top N are closed under ancestors).  Order: score desc, depth asc,
    tuple asc; the score is the float64 product taken from depth 1 down.
    The fixed rule of the tree module is the case q[d][r] = decay**(d+1)/(r+1).
  * The budget N itself is chosen by expected tokens per second, the expected
    tokens of the N-tree over the measured step time at that N.
"""

from itertools import product

import numpy as np

from .tree import TreePlan

MAX_K = 16   # shortlist size per head (columns of q)


def _score(t, q):
    s = 1.0
    for d, r in enumerate(t):
        s = s * float(q[d][r])
    return s


def _plan_of(nodes):
    index = {t: i for i, t in enumerate(nodes)}
    T = len(nodes)
    parent = np.full(T, -1, dtype=np.int64)
    depth = np.zeros(T, dtype=np.int64)
    for i, t in enumerate(nodes[1:], start=1):
        parent[i] = index[t[:-1]]
        depth[i] = len(t)
    anc = np.zeros((T, T), dtype=bool)
    for i in range(T):
        j = i
        while j >= 0:
            anc[i, j] = True
            j = parent[j]
    return TreePlan(tuples=nodes, parent=parent, depth=depth, anc=anc)


def expected_tokens(plan, q):
    """1 + sum over candidates (node order) of prod_d q[d][r_d]."""
    e = 1.0
    for t in plan.tuples[1:]:
        e = e + _score(t, q)
    return e


def tree_plan_rates(k, N, q):
    """(plan, expected tokens) of the N-candidate tree with the largest path
    acceptance products; N = None keeps every tuple."""
    k = list(k)
    tuples = []
    for D in range(1, len(k) + 1):
        tuples.extend(product(*[range(s) for s in k[:D]]))
    if N is None:
        kept = tuples
    else:
        if not 0 <= N <= len(tuples):
            raise ValueError("N exceeds the number of candidate tuples")
        ranked = sorted(tuples, key=lambda t: (-_score(t, q), len(t), t))
        kept = ranked[:N]
    nodes = [()] + sorted(kept, key=lambda t: (len(t), t))
    plan = _plan_of(nodes)
    return plan, expected_tokens(plan, q)


def plan_from_tables(k, parent, rank):
    """A tree given as parent and rank per node (node 0 the root).  Valid when
    every node's parent comes before it, depths never decrease along the node
    order, depth <= len(k), rank < k[depth-1] and no two children of one
    parent share a rank; raises ValueError otherwise."""
    parent = [int(p) for p in parent]
    rank = [int(r) for r in rank]
    if not parent or parent[0] != -1:
        raise ValueError("node 0 must be the root")
    tuples = [()]
    seen = set()
    for i in range(1, len(parent)):
        p = parent[i]
        if not 0 <= p < i:
            raise ValueError("parent must precede the node")
        t = tuples[p] + (rank[i],)
        if len(t) > len(k) or not 0 <= rank[i] < k[len(t) - 1]:
            raise ValueError("rank out of range")
        if len(t) < len(tuples[-1]):
            raise ValueError("depths must not decrease along the node order")
        if t in seen:
            raise ValueError("two children share a rank")
        seen.add(t)
        tuples.append(t)
    return _plan_of(tuples)


def accept_tally(plan, K, L, path):
    """Counts over one batch of steps: accepted[d][r] += 1 for the node of
    depth d+1 and rank r on the accepted path; offered[d][r] += 1 for every
    node of depth d+1 whose parent lies on the accepted path at depth d
    (d + 1 <= L + 1).  L: [b]; path: [b, K+1] node indices."""
    acc = np.zeros((K, MAX_K), dtype=np.int64)
    off = np.zeros((K, MAX_K), dtype=np.int64)
    for s in range(len(L)):
        Ls = int(L[s])
        if not 0 <= Ls <= K:
            continue
        on_path = {int(path[s][d]): d for d in range(Ls + 1)}
        for i in range(1, plan.T):
            t = plan.tuples[i]
            D = len(t)
            p = int(plan.parent[i])
            if p in on_path and on_path[p] == D - 1:
                off[D - 1][t[-1]] += 1
                if D <= Ls and int(path[s][D]) == i:
                    acc[D - 1][t[-1]] += 1
    return acc, off
