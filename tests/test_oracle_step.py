"""Whole-step oracle run on the tiny workload, and planted-mistake checks.

The planted mistakes live in the oracle only (monkeypatched copies on the
CPU): each must make at least one pin fail, which shows that the pins would
catch that kind of slip (wrong sign, transposed operand, dropped term, wrong
index).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import oracle_step, tree_plan, tree_attention, path_attention
import importlib

oracle_heads_mod = importlib.import_module("oracle.heads")
from speculative_decoding_heads_amd.configs import TINY, LLAMA7B_BS1
from speculative_decoding_heads_amd.synth import make_inputs


def _np(t):
    return t.float().numpy().astype(np.float64)


def test_tiny_step_runs_and_is_consistent():
    cfg = TINY
    x = {k: _np(v) for k, v in make_inputs(cfg).items()}
    P = np.full(cfg.b, cfg.P)
    out = oracle_step(x["h"], x["W"], x["LM"], x["Q"], x["Kc"], x["Vc"], P, cfg.k, cfg.N,
                      cfg.decay, cfg.mode, bf16=False)
    assert out["logits"].shape == (1, 4, cfg.V)
    assert out["tokens"].shape == (1, 11)
    assert out["O"].shape == (1, 11, cfg.nq * cfg.d)
    L = int(out["L"][0])
    assert 0 <= L <= cfg.K and out["seq_len"][0] == cfg.P + L + 1
    # the root is the base head's argmax; shortlists are distinct per head
    assert out["root"][0] == np.argmax(out["logits"][0, 0])
    for i in range(cfg.K):
        sl = out["idx"][0, i, : cfg.k[i]]
        assert len(set(sl.tolist())) == cfg.k[i]


def test_synth_is_deterministic_and_shaped():
    a = make_inputs(TINY, names=("h", "Q"))
    b = make_inputs(TINY, names=("h", "Q"))
    assert all(bool((a[k] == b[k]).all()) for k in a)
    assert tuple(a["Q"].shape) == (1, 11, 4, 64)
    w = make_inputs(LLAMA7B_BS1.with_(H=64, V=128), names=("LM",))["LM"]
    assert str(w.dtype) == "torch.bfloat16" and abs(float(w.float().std()) - 0.02) < 0.003


# ------------------------------------------------------------ planted mistakes
def _pins_fail(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_transposed_head_weight_is_caught(monkeypatch):
    import tests.test_oracle_numerics as tn
    orig = oracle_heads_mod.head_hidden

    def bad(h, W, bf16):
        return orig(h, None if W is None else np.transpose(W, (0, 2, 1)), bf16)

    monkeypatch.setattr(oracle_heads_mod, "head_hidden", bad)
    assert _pins_fail(tn.test_heads_against_python_loops)


def test_planted_silu_sign_is_caught(monkeypatch):
    import tests.test_oracle_numerics as tn
    monkeypatch.setattr(oracle_heads_mod, "silu", lambda z: z / (1.0 + np.exp(z)))
    assert _pins_fail(tn.test_heads_against_python_loops)


def test_planted_missing_self_in_mask_is_caught():
    plan = tree_plan((2, 2), None)
    rng = np.random.default_rng(0)
    Q = rng.standard_normal((1, plan.T, 2, 8))
    Kc = rng.standard_normal((1, 2, 5 + plan.T, 8))
    Vc = rng.standard_normal((1, 2, 5 + plan.T, 8))
    bad = plan.anc & ~np.eye(plan.T, dtype=bool)
    a = tree_attention(Q, Kc, Vc, [5], bad)
    b = path_attention(Q, Kc, Vc, [5], plan.parent)
    assert not np.allclose(a, b)


def test_planted_tree_score_exponent_is_caught(monkeypatch):
    ot = importlib.import_module("oracle.tree")
    import tests.test_oracle_tree as tt
    from fractions import Fraction

    def bad_score(t, decay):          # decay**1 at every depth instead of decay**d
        s = Fraction(1)
        for r in t:
            s *= decay / (r + 1)
        return s

    monkeypatch.setattr(ot, "tuple_score", bad_score)
    assert _pins_fail(lambda: tt.test_large_sparse_plans_match_hand_derivation(
        "tree_k10x4_n64.txt", (10,) * 4, 64))


def _hand_step_inputs():
    """A step small enough to work out by hand (hidden 4, vocab 6, K = 2,
    shortlists (2, 1) as a full tree, one attention head of dim 4, prefix 1).

    h = e0.  Head 1 has W_1[1, 0] = 20 and head 2 has W_2[2, 0] = 20, the
    rest zero, so u_1 = e0 + SiLU(20) e1 and u_2 = e0 + SiLU(20) e2 with
    SiLU(20) = 20 / (1 + e^-20) (within 5e-8 of 20).  LM columns:
      LM[:, 0] = (0.1, 0.5, 0.3, 0.9, 0.2, 0.4)   base head: argmax 3
      LM[:, 1] = (0,   0,   0.2, 0,   0.1, 0)     head 1 = LM[:,0] + ~20 LM[:,1]
                                                   = (0.1, 0.5, 4.3, 0.9, 2.2, 0.4)
      LM[:, 2] = (0.3, 0,   0,   0,   0,   0)     head 2 = (6.1, 0.5, 0.3, 0.9, 0.2, 0.4)
    Root = 3; head 1's top-2 = (2, 4); head 2's top-1 = (0,).  Tree (node
    order root, depth 1 by rank, depth 2 by rank tuple): node 1 = (0) token
    2, node 2 = (1) token 4, node 3 = (0, 0) token 0, node 4 = (1, 0) token 0;
    parents (-, 0, 0, 1, 2).  Tokens (3, 2, 4, 0, 0), positions P + depth.
    Attention with q = 0 averages the visible V rows (prefix slot and the
    path): V prefix = 0, V(node 0) = 10 e1, V(node 1) = 100 e2, V(node 3) =
    1000 e0, V(nodes 2, 4) = e3.
      o_0 = 10 e1 / 2         -> LM o_0 = (0, 0, 1, 0, 0.5, 0)        argmax 2
      o_1 = (10 e1 + 100 e2)/3 -> (30, 0, 2, 0, 1, 0) / 3            argmax 0
      o_3 = (10 e1 + 100 e2 + 1000 e0)/4
                               -> (130, 500, 302, 900, 201, 400) / 4 argmax 3
    Greedy walk: root's argmax 2 = node 1's token -> node 1; node 1's
    argmax 0 = node 3's token -> node 3 (depth 2 = K, a leaf): L = 2, path
    (0, 1, 3), accepted tokens (3, 2, 0), next token = argmax at node 3 = 3.
    Compaction: slot P+2 takes slot P+3; seq_len = P + 3.
    """
    H, V = 4, 6
    h = np.zeros((1, H))
    h[0, 0] = 1.0
    W = np.zeros((2, H, H))
    W[0, 1, 0] = 20.0
    W[1, 2, 0] = 20.0
    LM = np.zeros((V, H))
    LM[:, 0] = [0.1, 0.5, 0.3, 0.9, 0.2, 0.4]
    LM[:, 1] = [0, 0, 0.2, 0, 0.1, 0]
    LM[:, 2] = [0.3, 0, 0, 0, 0, 0]
    P, T = 1, 5
    Q = np.zeros((1, T, 1, H))
    Kc = np.arange(1 * 1 * (P + T) * H, dtype=np.float64).reshape(1, 1, P + T, H)
    Vc = np.zeros((1, 1, P + T, H))
    Vc[0, 0, P + 0, 1] = 10.0
    Vc[0, 0, P + 1, 2] = 100.0
    Vc[0, 0, P + 3, 0] = 1000.0
    Vc[0, 0, P + 2, 3] = 1.0
    Vc[0, 0, P + 4, 3] = 1.0
    return h, W, LM, Q, Kc, Vc, P


def test_hand_derived_step():
    h, W, LM, Q, Kc, Vc, P = _hand_step_inputs()
    out = oracle_step(h, W, LM, Q, Kc, Vc, np.array([P]), (2, 1), None, Fraction(4, 5), "greedy",
                      bf16=False)
    s20 = 20.0 / (1.0 + np.exp(-20.0))
    assert np.allclose(out["u"][0], [[1, 0, 0, 0], [1, s20, 0, 0], [1, 0, s20, 0]], atol=0)
    assert np.allclose(out["logits"][0, 1], [0.1, 0.5, 0.3 + 0.2 * s20, 0.9, 0.2 + 0.1 * s20,
                                             0.4], atol=1e-15)
    assert out["root"][0] == 3
    assert list(out["idx"][0, 0, :2]) == [2, 4] and out["idx"][0, 1, 0] == 0
    assert list(out["plan"].parent) == [-1, 0, 0, 1, 2]
    assert list(out["tokens"][0]) == [3, 2, 4, 0, 0]
    assert list(out["pos"][0]) == [1, 2, 2, 3, 3]
    O = out["O"][0]
    assert np.allclose(O[0], [0, 5, 0, 0], atol=1e-12)
    assert np.allclose(O[1], [0, 10 / 3, 100 / 3, 0], atol=1e-12)
    assert np.allclose(O[3], [250, 2.5, 25, 0], atol=1e-12)
    assert np.allclose(out["base_logits"][0, 3], np.array([130, 500, 302, 900, 201, 400]) / 4,
                       atol=1e-12)
    assert out["L"][0] == 2
    assert list(out["path"][0]) == [0, 1, 3]
    assert list(out["acc_tokens"][0]) == [3, 2, 0]
    assert out["bonus"][0] == 3
    assert out["seq_len"][0] == P + 3
    assert np.array_equal(out["Kc"][0, 0, P + 2], Kc[0, 0, P + 3])
    assert np.array_equal(out["Vc"][0, 0, P + 2], Vc[0, 0, P + 3])
    assert np.array_equal(out["Kc"][0, 0, : P + 2], Kc[0, 0, : P + 2])


def test_hand_derived_step_catches_a_head_index_slip(monkeypatch):
    # planted mistake (oracle only, on the CPU): head 1's shortlist taken from
    # the base head's logits, i.e. logits[s, i] in place of logits[s, i + 1]
    import oracle.step as step_mod
    real = step_mod.topk_stable
    h, W, LM, Q, Kc, Vc, P = _hand_step_inputs()
    base_row = LM @ h[0]
    calls = []

    def slip(row, k):
        calls.append(k)
        return real(base_row if len(calls) == 1 else row, k)

    monkeypatch.setattr(step_mod, "topk_stable", slip)
    assert _pins_fail(test_hand_derived_step)
