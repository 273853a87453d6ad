"""One full draft-and-verify step, chaining the oracle stages (test infra).

Order of the decoding loop (inferensys.com "Medusa Heads", the loop of
drafting, verification, acceptance and rollback):
  1. heads: base head + K Medusa heads from one hidden state per sequence;
  2. shortlists: top-k_i per Medusa head, root = the base head's token;
  3. tree: fixed sparse tree, gathered tokens and position ids;
  4. verification: tree-masked attention over prefix + tree;
  5. the base model's original output head on each node (here the shared
     LM projection of the attention output; one-layer stand-in for the
     backbone's verify pass, n_q * d = H);
  6. acceptance (greedy or typical) and the next token;
  7. compaction of the accepted path's K/V entries.
"""

import numpy as np

from .heads import heads, lm_project
from .topk import topk_stable, argmax_lowest
from .rng import counter_uniform, sample_tempered
from .tree import tree_plan, tree_gather
from .attention import tree_attention
from .accept import accept_greedy_walk, accept_greedy_parallel, accept_typical, accept_reject
from .compact import kv_compact


def oracle_step(h, W, LM, Q, Kc, Vc, P, k, N, decay, mode, bf16,
                temperature=1.0, eps=0.3, delta=0.09, seed=0, step=0, plan=None):
    b = h.shape[0]
    K = len(k)
    kmax = max(k)
    u, logits = heads(h, W, LM, bf16)
    root = np.empty(b, dtype=np.int64)
    idx = np.full((b, K, kmax), -1, dtype=np.int64)
    for s in range(b):
        if mode == "greedy":
            root[s] = argmax_lowest(logits[s, 0])
        else:
            root[s], _ = sample_tempered(logits[s, 0], temperature,
                                         counter_uniform(seed, step, s, 0))
        for i in range(K):
            idx[s, i, : k[i]] = topk_stable(logits[s, i + 1], k[i])
    if plan is None:
        plan = tree_plan(k, N, decay)
    T = plan.T
    tokens = np.empty((b, T), dtype=np.int64)
    pos = np.empty((b, T), dtype=np.int64)
    for s in range(b):
        tokens[s], pos[s] = tree_gather(plan, root[s], idx[s], int(P[s]))
    O = tree_attention(Q, Kc, Vc, P, plan.anc, bf16=bf16)
    H = O.shape[-1]
    base_logits = lm_project(O.reshape(b * T, H), LM).reshape(b, T, -1)
    L = np.empty(b, dtype=np.int64)
    path = np.empty((b, K + 1), dtype=np.int64)
    acc = np.empty((b, K + 1), dtype=np.int64)
    bonus = np.empty(b, dtype=np.int64)
    Kn = np.array(Kc, copy=True)
    Vn = np.array(Vc, copy=True)
    new_len = np.empty(b, dtype=np.int64)
    for s in range(b):
        if mode == "greedy":
            L[s], path[s], acc[s], bonus[s] = accept_greedy_walk(
                base_logits[s], tokens[s], plan.parent, K)
            chk = accept_greedy_parallel(base_logits[s], tokens[s], plan.parent, plan.depth, K)
            assert chk[0] == L[s] and (chk[1] == path[s]).all() and chk[3] == bonus[s]
        elif mode == "typical":
            L[s], path[s], acc[s], bonus[s], _ = accept_typical(
                base_logits[s], tokens[s], plan.parent, plan.depth, K,
                temperature, eps, delta, seed, step, s)
        elif mode == "reject":
            L[s], path[s], acc[s], bonus[s], _ = accept_reject(
                base_logits[s], tokens[s], plan.parent, K, temperature, seed, step, s)
        else:
            raise ValueError(f"unknown acceptance mode {mode!r}")
        Kn[s], Vn[s], new_len[s] = kv_compact(Kc[s], Vc[s], int(P[s]), path[s], int(L[s]))
    return dict(u=u, logits=logits, root=root, idx=idx, plan=plan, tokens=tokens,
                pos=pos, O=O, base_logits=base_logits, L=L, path=path,
                acc_tokens=acc, bonus=bonus, Kc=Kn, Vc=Vn, seq_len=new_len)
