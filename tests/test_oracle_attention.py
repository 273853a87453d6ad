"""Pins for the oracle's tree attention.

inferensys.com "Medusa Heads" (tree attention over a shared prefix KV cache)
and zackli.ai "Speculative Decoding Deep Dive II" (Anc(i)): tree-masked
attention must equal plain causal attention over each root-to-node path taken
as its own sequence after the prefix.  Further pins: torch's
scaled_dot_product_attention on chains, and closed forms.
"""

import numpy as np
import torch
from hypothesis import given, settings, strategies as st

from oracle import tree_plan, tree_attention, path_attention
from oracle.attention import attention_row


def _inputs(b, T, nq, nkv, d, P, seed, extra=3):
    rng = np.random.default_rng(seed)
    Pmax = P + T + extra
    Q = rng.standard_normal((b, T, nq, d))
    Kc = rng.standard_normal((b, nkv, Pmax, d))
    Vc = rng.standard_normal((b, nkv, Pmax, d))
    return Q, Kc, Vc


@settings(max_examples=40, deadline=None)
@given(k=st.lists(st.integers(1, 4), min_size=1, max_size=3),
       frac=st.floats(0.0, 1.0), P=st.integers(0, 16),
       heads=st.sampled_from([(1, 1), (2, 2), (4, 2), (4, 1), (6, 3)]),
       seed=st.integers(0, 10 ** 6))
def test_masked_tree_equals_per_path_causal(k, frac, P, heads, seed):
    from oracle import full_tree_node_count
    N = int(round(frac * full_tree_node_count(k)))
    plan = tree_plan(k, N)
    nq, nkv = heads
    Q, Kc, Vc = _inputs(2, plan.T, nq, nkv, 8, P, seed)
    Pv = np.array([P, max(P - 1, 0)])
    a = tree_attention(Q, Kc, Vc, Pv, plan.anc)
    bb = path_attention(Q, Kc, Vc, Pv, plan.parent)
    assert np.allclose(a, bb, rtol=1e-12, atol=1e-12)


def test_workload_tree_masked_equals_paths():
    plan = tree_plan((10,) * 4, 64)
    Q, Kc, Vc = _inputs(1, plan.T, 2, 1, 16, 20, 5)
    a = tree_attention(Q, Kc, Vc, [20], plan.anc)
    bb = path_attention(Q, Kc, Vc, [20], plan.parent)
    assert np.allclose(a, bb, rtol=1e-12, atol=1e-12)


def test_root_only_without_prefix_returns_root_value():
    plan = tree_plan((2,), 0)
    Q, Kc, Vc = _inputs(1, 1, 2, 2, 8, 0, 6)
    O = tree_attention(Q, Kc, Vc, [0], plan.anc).reshape(1, 1, 2, 8)
    assert np.allclose(O[0, 0], Vc[0, :, 0], rtol=0, atol=1e-15)


def test_zero_query_averages_visible_values():
    plan = tree_plan((2, 2), None)
    P = 5
    Q, Kc, Vc = _inputs(1, plan.T, 1, 1, 4, P, 7)
    Q[:] = 0.0
    O = tree_attention(Q, Kc, Vc, [P], plan.anc).reshape(plan.T, 4)
    for t in range(plan.T):
        vis = list(range(P)) + [P + j for j in range(plan.T) if plan.anc[t, j]]
        assert np.allclose(O[t], Vc[0, 0, vis].mean(axis=0), atol=1e-14)


def test_chain_tree_is_standard_causal_attention():
    # k = (1,1,1): the tree is one chain; every node is position P+depth of one
    # causal sequence.  Compare with torch's SDPA (float64, causal).
    plan = tree_plan((1, 1, 1), None)
    P, nq, nkv, d = 7, 4, 2, 8
    Q, Kc, Vc = _inputs(1, plan.T, nq, nkv, d, P, 8, extra=0)
    O = tree_attention(Q, Kc, Vc, [P], plan.anc).reshape(plan.T, nq, d)
    L = P + plan.T
    rng = np.random.default_rng(99)
    qfull = rng.standard_normal((nq, L, d))
    qfull[:, P:, :] = np.transpose(Q[0], (1, 0, 2))
    k = torch.from_numpy(Kc[0]).repeat_interleave(nq // nkv, dim=0)
    v = torch.from_numpy(Vc[0]).repeat_interleave(nq // nkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qfull), k, v, is_causal=True)
    assert np.allclose(O, ref.numpy()[:, P:, :].transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_gqa_head_mapping():
    # q head h reads kv head floor(h * nkv / nq): move kv head 1's data and
    # only q heads 2,3 (of 4, nkv = 2) may change.
    plan = tree_plan((2,), None)
    Q, Kc, Vc = _inputs(1, plan.T, 4, 2, 8, 3, 9)
    a = tree_attention(Q, Kc, Vc, [3], plan.anc).reshape(plan.T, 4, 8)
    Vc2 = Vc.copy()
    Vc2[:, 1] += 1.0
    c = tree_attention(Q, Kc, Vc2, [3], plan.anc).reshape(plan.T, 4, 8)
    assert np.allclose(a[:, :2], c[:, :2], atol=0)
    assert np.allclose(c[:, 2:], a[:, 2:] + 1.0, atol=1e-12)


def test_sampled_row_helper_matches_batch_routine():
    plan = tree_plan((3, 2), 5)
    Q, Kc, Vc = _inputs(1, plan.T, 2, 1, 8, 6, 10)
    O = tree_attention(Q, Kc, Vc, [6], plan.anc).reshape(plan.T, 2, 8)
    for t in range(plan.T):
        r = attention_row(Q[0, t, 1], Kc[0, 0], Vc[0, 0], 6, plan.anc[t], 1 / np.sqrt(8))
        assert np.allclose(r, O[t, 1], atol=1e-14)


@settings(max_examples=30, deadline=None)
@given(k=st.lists(st.integers(1, 4), min_size=1, max_size=3), frac=st.floats(0.0, 1.0),
       P=st.integers(0, 12), heads=st.sampled_from([(2, 2), (4, 2), (6, 3)]),
       seed=st.integers(0, 10 ** 6))
def test_head_matrix_form_equals_per_path_causal(k, frac, P, heads, seed):
    # the score-matrix form used by the full-size checks (one q head, every
    # node) must equal the brute-force per-path causal attention
    from oracle import full_tree_node_count
    from oracle.attention import tree_attention_head
    N = int(round(frac * full_tree_node_count(k)))
    plan = tree_plan(k, N)
    nq, nkv = heads
    d = 8
    Q, Kc, Vc = _inputs(1, plan.T, nq, nkv, d, P, seed)
    ref = path_attention(Q, Kc, Vc, [P], plan.parent).reshape(plan.T, nq, d)
    G = nq // nkv
    for hq in range(nq):
        got = tree_attention_head(Q[0, :, hq], Kc[0, hq // G], Vc[0, hq // G], P, plan.anc,
                                  1 / np.sqrt(d))
        assert np.allclose(got, ref[:, hq], rtol=1e-12, atol=1e-12)
