"""Consecutive steps with the state carried on the device (VerifyLoop).

Each step's arithmetic is checked stage by stage elsewhere; here the state that
moves between steps is checked exactly, and every step's discrete outcome is
checked against the oracle deciding on the GPU's own floats:
  * the tree K/V of step s land at slots P_s .. P_s+T-1 (a CPU model of the
    cache applies the same appends and the oracle's compaction, and must equal
    the GPU cache bit for bit at the end);
  * shortlists / tree tokens / positions: the oracle's stable top-k and tree
    gather on the GPU's head logits, with the root of step s >= 1 equal to the
    next token of step s-1;
  * attention output of each step within tolerance of the oracle on the CPU
    cache model (small workloads);
  * acceptance (L, path, next token) by the oracle on the GPU's verify logits;
  * seq_len advances by L + 1, and the next hidden state is the chosen node's
    attention output row, bit for bit.
A HIP graph of the whole loop, replayed three times from the same start state
with eager work in between, must reproduce the eager run bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle.accept import accept_greedy_walk, accept_typical
from oracle.attention import tree_attention
from oracle.compact import kv_compact
from oracle.topk import argmax_lowest, topk_stable
from oracle.tree import tree_gather, tree_plan
from speculative_decoding_heads_amd import configs as C
from speculative_decoding_heads_amd.step import VerifyLoop, device_inputs, loop_inputs
from speculative_decoding_heads_amd.synth import make_inputs
from tests.helpers import TOL_BF16, TOL_F32, np64, require_gpu, row_rel_err, say

pytestmark = pytest.mark.gpu

STEPS = 4
LOOP = [
    C.Config("loop_bf16_greedy", 95, 2, 256, 3000, (4, 3, 2), 20, 4, 2, 64, 300, "bf16", "greedy"),
    C.Config("loop_bf16_typical", 96, 2, 384, 5000, (5, 4, 3), 40, 6, 3, 64, 200, "bf16",
             "typical"),
    C.Config("loop_f32_greedy", 97, 1, 256, 4096, (2, 2, 1), None, 4, 4, 64, 128, "f32", "greedy",
             temperature=1.0),
    C.LLAMA7B_BS1,
]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _state(cfg, steps):
    """Device state with a cache large enough for `steps` steps (prefix copied)."""
    host = make_inputs(cfg)
    x = device_inputs(cfg, host)
    cap = cfg.P + steps * (cfg.K + 1) + cfg.T
    for name in ("Kc", "Vc"):
        big = torch.zeros(cfg.b, cfg.nkv, cap, cfg.d, dtype=x[name].dtype, device="cuda")
        big[:, :, : cfg.P] = x[name][:, :, : cfg.P]
        x[name] = big
    return x


def _clone(x):
    return {k: v.clone() for k, v in x.items()}


def _run_eager(cfg, x, Qs, Kn, Vn):
    loop = VerifyLoop(cfg)
    st = loop.step
    rec = []

    def after(s):
        torch.cuda.synchronize()
        rec.append({k: getattr(st, k).clone() for k in
                    ("logits", "tokens", "pos", "O", "base_logits", "L", "path", "bonus")}
                   | {"h": x["h"].clone(), "seq_len": x["seq_len"].clone()})

    loop.run(x, Qs, Kn, Vn, after_step=after)
    torch.cuda.synchronize()
    return rec


@pytest.mark.parametrize("cfg", LOOP, ids=lambda c: c.name)
def test_loop_state_and_decisions(cfg):
    say("loop", cfg.name, STEPS)
    x = _state(cfg, STEPS)
    x0 = {k: np64(v) for k, v in x.items() if k in ("Kc", "Vc", "seq_len")}
    Qs, Kn, Vn = loop_inputs(cfg, STEPS, seed_base=cfg.index)
    rec = _run_eager(cfg, x, Qs, Kn, Vn)
    plan = tree_plan(cfg.k, cfg.N, cfg.decay)
    K, T = cfg.K, cfg.T
    Kcpu, Vcpu = x0["Kc"].copy(), x0["Vc"].copy()
    P = x0["seq_len"].astype(np.int64)
    Kn64, Vn64 = np64(Kn), np64(Vn)
    small = cfg.H <= 512
    for s, r in enumerate(rec):
        for q in range(cfg.b):                              # the append
            Kcpu[q, :, P[q]:P[q] + T] = Kn64[s, q]
            Vcpu[q, :, P[q]:P[q] + T] = Vn64[s, q]
        logits = np64(r["logits"])
        tokens = r["tokens"].cpu().numpy()
        for q in range(cfg.b):
            if s == 0:
                root = argmax_lowest(logits[q, 0]) if cfg.mode == "greedy" else tokens[q, 0]
            else:
                root = int(rec[s - 1]["bonus"][q])
            idx = np.full((K, cfg.kmax), -1, dtype=np.int64)
            for i in range(K):
                idx[i, : cfg.k[i]] = topk_stable(logits[q, i + 1], cfg.k[i])
            want_t, want_p = tree_gather(plan, int(root), idx, int(P[q]))
            assert list(tokens[q]) == list(want_t), (s, q)
            assert list(r["pos"][q].cpu().numpy()) == list(want_p), (s, q)
        if small:
            ref = tree_attention(np64(Qs[s]), Kcpu, Vcpu, P, plan.anc, bf16=cfg.dtype == "bf16")
            got = np64(r["O"]).reshape(ref.shape)
            tol = TOL_BF16 if cfg.dtype == "bf16" else TOL_F32
            assert row_rel_err(got, ref) <= tol, s
        base = np64(r["base_logits"])
        L = r["L"].cpu().numpy()
        path = r["path"].cpu().numpy()
        bonus = r["bonus"].cpu().numpy()
        for q in range(cfg.b):
            if cfg.mode == "greedy":
                wL, wpath, _, wb = accept_greedy_walk(base[q], tokens[q], plan.parent, K)
                guarded = False
            else:
                wL, wpath, _, wb, margins = accept_typical(
                    base[q], tokens[q], plan.parent, plan.depth, K,
                    float(np.float32(cfg.temperature)), float(np.float32(cfg.eps)),
                    float(np.float32(cfg.delta)), cfg.seed, s, q)
                guarded = np.min(margins[1:]) < 1e-4
            if not guarded:
                assert L[q] == wL and list(path[q]) == list(wpath), (s, q)
                if cfg.mode == "greedy":
                    assert bonus[q] == wb, (s, q)
            Kq, Vq, newP = kv_compact(Kcpu[q], Vcpu[q], int(P[q]), path[q], int(L[q]))
            Kcpu[q], Vcpu[q] = Kq, Vq
            assert int(r["seq_len"][q]) == newP == P[q] + L[q] + 1, (s, q)
            P[q] = newP
            # next hidden state = the chosen node's verification state
            node = int(path[q, L[q]])
            assert torch.equal(r["h"][q].reshape(-1), r["O"][q, node].reshape(-1)), (s, q)
    assert np.array_equal(np64(x["Kc"]), Kcpu) and np.array_equal(np64(x["Vc"]), Vcpu)


@pytest.mark.parametrize("cfg", [LOOP[1], C.LLAMA7B_BS1], ids=lambda c: c.name)
def test_loop_graph_replays_match_eager(cfg):
    say("loop graph", cfg.name, STEPS)
    x_init = _state(cfg, STEPS)
    Qs, Kn, Vn = loop_inputs(cfg, STEPS, seed_base=cfg.index)
    xe = _clone(x_init)
    loop_e = VerifyLoop(cfg)
    loop_e.run(xe, Qs, Kn, Vn)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in xe.items()}
    ref_out = {k: getattr(loop_e.step, k).clone() for k in ("tokens", "L", "path", "bonus", "O")}

    xg = _clone(x_init)
    loop_g = VerifyLoop(cfg)
    g = loop_g.capture(xg, Qs, Kn, Vn)
    for rep in range(3):
        for k in xg:                                     # eager reset between replays
            xg[k].copy_(x_init[k])
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("h", "Kc", "Vc", "seq_len"):
            assert torch.equal(xg[k], ref[k]), (rep, k)
        for k, v in ref_out.items():
            assert torch.equal(getattr(loop_g.step, k), v), (rep, k)
        del junk
