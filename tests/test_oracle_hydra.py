"""Pins of the Hydra-style draft oracle (oracle/hydra.py) against what the
pages and the mathematics fix, independently of its own loop:

  * with a zero embedding table the draft is the Medusa draft: the K heads on
    h_t, one shortlist per head, and the tree gather (zackli.ai "Speculative
    Decoding Deep Dive II", "Medusa": Hydra differs from Medusa only in feeding
    the drafted token to the later heads);
  * a closed form: with h = 0, W = 0 and LM = I, head d returns e(x) for the
    parent token x, so an embedding table that puts its peak at pi(x) and
    falls off with (v - pi(x)) mod V gives token(child of rank r) =
    (pi(x) + r) mod V down every path -- each head sees exactly its parent's
    token;
  * a head sees only its parent's token: changing the token of one depth-1
    node changes the tokens below it and nothing else.
"""

import numpy as np
import pytest

from oracle import heads, hydra_draft, round_bf16, topk_stable, tree_gather, tree_plan


def _weights(H, V, K, seed):
    rng = np.random.default_rng(seed)
    h = round_bf16(rng.standard_normal(H))
    W = round_bf16(rng.normal(0.0, 0.05, size=(K, H, H)))
    LM = round_bf16(rng.normal(0.0, 0.05, size=(V, H)))
    E = round_bf16(rng.normal(0.0, 0.5, size=(V, H)))
    return h, W, LM, E


@pytest.mark.parametrize("k,N,bf16", [((3, 2, 2), None, True), ((4, 3, 2), 12, False),
                                      ((10, 10, 10, 10), 64, True)])
def test_zero_embedding_is_the_medusa_draft(k, N, bf16):
    H, V = 64, 300
    K = len(k)
    h, W, LM, _ = _weights(H, V, K, 11 + K)
    plan = tree_plan(k, N)
    _, logits = heads(h[None, :], W, LM, bf16)
    root = int(np.argmax(logits[0, 0]))
    idx = np.zeros((K, max(k)), dtype=np.int64)
    for i in range(K):
        idx[i, : k[i]] = topk_stable(logits[0, i + 1], k[i])
    want, _ = tree_gather(plan, root, idx, 0)
    got, rows = hydra_draft(h, np.zeros((V, H)), W, LM, k, plan, root, bf16=bf16)
    assert list(got) == list(want)
    for p, row in rows.items():       # every parent of a depth saw the same head logits
        d = int(plan.depth[p]) + 1
        assert np.allclose(row, logits[0, d], rtol=0, atol=1e-12)


def test_permutation_embedding_closed_form():
    V = H = 16
    k = (3, 2, 2, 2)
    K = len(k)
    plan = tree_plan(k, None)
    pi = np.random.default_rng(5).permutation(V)
    E = np.zeros((V, H))
    for x in range(V):
        for v in range(V):
            m = (v - pi[x]) % V
            E[x, v] = 1.0 if m == 0 else -0.001 * m
    E = round_bf16(E)
    root = 7
    got, _ = hydra_draft(np.zeros(H), E, np.zeros((K, H, H)), np.eye(V), k, plan, root)
    want = {(): root}
    for t in sorted(plan.tuples, key=len)[1:]:
        want[t] = (pi[want[t[:-1]]] + t[-1]) % V
    assert [int(x) for x in got] == [int(want[t]) for t in plan.tuples]


def test_a_head_sees_only_its_parents_token():
    H, V = 64, 200
    k = (3, 3, 2)
    K = len(k)
    h, W, LM, E = _weights(H, V, K, 3)
    plan = tree_plan(k, None)
    base, _ = hydra_draft(h, E, W, LM, k, plan, 9)
    forced = base.copy()
    forced[1] = (base[1] + 17) % V        # another token at node 1 (depth 1)
    got, _ = hydra_draft(h, E, W, LM, k, plan, 9, parent_tokens=forced)
    below = {c for c in range(plan.T) if plan.anc[c, 1] and c != 1}
    for c in range(1, plan.T):
        if c in below:
            continue
        assert got[c] == base[c], c
    assert any(got[c] != base[c] for c in below)
