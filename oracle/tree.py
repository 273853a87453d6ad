"""Sparse candidate tree, its ancestor mask and per-step gather (oracle).

Test infrastructure only.

Pages:
  * aicassindra.com "Medusa deep dive", "From top-k heads to a sparse candidate
    tree": the Cartesian product of per-head shortlists is pruned to a fixed
    sparse tree chosen ahead of time, giving more branches to confident, early
    heads; the tree is laid out as a flat node sequence with a matching
    attention mask and position ids, and a node attends only to its ancestors.
  * zackli.ai "Speculative Decoding Deep Dive II", section "Medusa": Anc(i) is
    the set of ancestors of node i; with shortlist sizes s_1, s_2, ... there
    are s_1*s_2*... full paths and s_1 + s_1*s_2 + s_1*s_2*s_3 + ... tree nodes.

Readings (the pages fix no ranking rule, order or root convention):
  * A node below the root is a rank tuple (r_1, ..., r_D), 1 <= D <= K,
    0 <= r_d < k_d: the candidate takes rank r_d of head d at depth d.
  * Sparse selection score: prod_{d=1..D} decay**d / (r_d + 1) with
    decay = 4/5, compared exactly (Fractions); order (score desc, D asc,
    tuple lexicographic asc); keep the first N.  A child always scores strictly
    below its parent, so the kept set is closed under taking ancestors.
  * N counts the candidates only; the root (the base head's token) is node 0,
    T = N + 1 nodes in all.
  * Flat order: root, then by depth, lexicographic by rank tuple within a
    depth.  Hence parent index < child index.
  * Mask row i marks i itself and every ancestor of i (the root included).
  * Position id of node i = P + depth(i) for a prefix of length P.
"""

from dataclasses import dataclass
from fractions import Fraction
from itertools import product

import numpy as np


def full_tree_node_count(k):
    """s_1 + s_1 s_2 + s_1 s_2 s_3 + ...  (candidates only, root excluded)."""
    total, prod_ = 0, 1
    for s in k:
        prod_ *= s
        total += prod_
    return total


def full_path_count(k):
    """s_1 * s_2 * ... : root-to-leaf paths of the full tree."""
    p = 1
    for s in k:
        p *= s
    return p


def tuple_score(t, decay):
    """prod_{d=1..D} decay**d / (r_d + 1) as an exact Fraction."""
    s = Fraction(1)
    for d, r in enumerate(t, start=1):
        s *= decay ** d / (r + 1)
    return s


@dataclass
class TreePlan:
    tuples: list          # node -> rank tuple (root: ())
    parent: np.ndarray    # [T] int64, -1 for the root
    depth: np.ndarray     # [T] int64
    anc: np.ndarray       # [T, T] bool; anc[i, j] = j is i or an ancestor of i

    @property
    def T(self):
        return len(self.tuples)


def tree_plan(k, N=None, decay=Fraction(4, 5)):
    """The fixed tree for shortlist sizes k (one per head) and N candidates.

    N = None keeps every tuple (the full tree).
    """
    k = list(k)
    decay = Fraction(decay)
    all_tuples = []
    for D in range(1, len(k) + 1):
        all_tuples.extend(product(*[range(s) for s in k[:D]]))
    if N is None:
        kept = all_tuples
    else:
        if not 0 <= N <= len(all_tuples):
            raise ValueError("N exceeds the number of candidate tuples")
        ranked = sorted(all_tuples, key=lambda t: (-tuple_score(t, decay), len(t), t))
        kept = ranked[:N]
    nodes = [()] + sorted(kept, key=lambda t: (len(t), t))
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


def tree_gather(plan, root, idx, P):
    """Per-step candidate tokens and position ids.

    token[0] = root; token[i] = idx[depth-1][last rank of node i], i.e. the
    r_D-th shortlist entry of head D.  pos[i] = P + depth[i].
    root: int; idx: [K, kmax] shortlist indices of one sequence.
    """
    T = plan.T
    tokens = np.empty(T, dtype=np.int64)
    tokens[0] = root
    for i in range(1, T):
        t = plan.tuples[i]
        tokens[i] = idx[len(t) - 1][t[-1]]
    pos = P + plan.depth.copy()
    return tokens, pos
