"""The largest shapes the library accepts, end to end on the GPU against the
oracle: K = 16 heads, a 16-wide first shortlist (kmax = 16), a 255-candidate
tree (T = 256 nodes, four ancestor words per node) planned from per-rank
acceptance rates so that it reaches depth 16, greedy acceptance of a
17-node path, and the KV compaction of that path.

Shortlists, root, tree tables and tokens must equal the oracle's stable top-k,
argmax and gather on that tree; L, path, accepted tokens and the next token
must equal the oracle's token-by-token greedy replay; the cache after
compaction must equal the oracle's compaction bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle import (accept_greedy_walk, argmax_lowest, kv_compact, plan_from_tables, topk_stable,
                    tree_gather)
from speculative_decoding_heads_amd import medusa as M
from tests.helpers import normal, require_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
I32 = dict(dtype=torch.int32, device=DEV)
K = 16
SHORT = (16, 4) + (2,) * 14


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _rates():
    q = np.zeros((K, 16))
    for d, s in enumerate(SHORT):
        q[d, 0] = 0.97
        q[d, 1:s] = 0.3 / np.arange(2, s + 1)
    return q


def _chain_end(plan):
    """Deepest node reached by rank 0 at every depth."""
    node = 0
    for d in range(K):
        kids = [c for c in range(1, plan.T) if plan.parent[c] == node and plan.tuples[c][-1] == 0]
        if not kids:
            break
        node = kids[0]
    return node


def test_max_heads_max_tree_greedy_step():
    b, V, P = 3, 3000, 40
    par, dep, rk, _ = M.medusa_tree_plan_rates(SHORT, 255, _rates())
    plan = plan_from_tables(SHORT, par, rk)
    T = plan.T
    assert T == 256 and max(plan.depth) == K
    say("maxsize", b, V, T)
    # shortlists, root and tree in one launch
    logits = normal((b, K + 1, V), 777, 1.0, torch.float32)
    Pd = torch.full((b,), P, **I32)
    root = torch.empty(b, **I32)
    idx = torch.empty(b, K, 16, **I32)
    val = torch.empty(b, K, 16, dtype=torch.float32, device=DEV)
    tokens, pos = torch.empty(b, T, **I32), torch.empty(b, T, **I32)
    parent, depth = torch.empty(T, **I32), torch.empty(T, **I32)
    anc = torch.empty(T, 4, dtype=torch.int64, device=DEV)
    ws = M.workspace(M.medusa_topk_workspace(b, K, V, 16))
    M.medusa_topk_tree_tables(logits.to(DEV), SHORT, 16, par, rk, M.GREEDY, 1.0, 1, 2, Pd, root, idx,
                              val, tokens, pos, parent, depth, anc, ws)
    torch.cuda.synchronize()
    assert list(parent.cpu().numpy()) == list(plan.parent)
    assert list(depth.cpu().numpy()) == list(plan.depth)
    a = anc.cpu().numpy().view(np.uint64)
    for i in range(T):
        for j in range(T):
            assert bool((int(a[i, j // 64]) >> (j % 64)) & 1) == bool(plan.anc[i, j])
    x = logits.numpy()
    i_gpu, r_gpu = idx.cpu().numpy(), root.cpu().numpy()
    tok = tokens.cpu().numpy()
    for s in range(b):
        assert r_gpu[s] == argmax_lowest(x[s, 0])
        for i in range(K):
            assert list(i_gpu[s, i, : SHORT[i]]) == list(topk_stable(x[s, i + 1], SHORT[i]))
        tk, ps = tree_gather(plan, int(r_gpu[s]), i_gpu[s], P)
        assert list(tok[s]) == list(tk) and list(pos[s].cpu().numpy()) == list(ps)
    # greedy acceptance: sequence 0 accepts the full rank-0 chain, sequence 1
    # stops at depth 9 on it, sequence 2 is left random
    base = normal((b, T, V), 778, 1.0, torch.float32).numpy()
    end = _chain_end(plan)
    chain = []
    n = end
    while n > 0:
        chain.append(n)
        n = int(plan.parent[n])
    chain = chain[::-1]
    assert len(chain) == K
    for s, stop in ((0, K), (1, 9)):
        for c in chain[:stop]:
            base[s, plan.parent[c], tok[s, c]] = 60.0
    Lg, path = torch.empty(b, **I32), torch.empty(b, K + 1, **I32)
    acc, bonus = torch.empty(b, K + 1, **I32), torch.empty(b, **I32)
    wsa = M.workspace(M.medusa_accept_workspace(b, T))
    M.medusa_accept(torch.from_numpy(base).to(DEV), tokens, parent, depth, K, M.GREEDY, 1.0, 0.3,
                    0.09, 0, 0, Lg, path, acc, bonus, wsa)
    torch.cuda.synchronize()
    Lh, ph, ah, bh = Lg.cpu().numpy(), path.cpu().numpy(), acc.cpu().numpy(), bonus.cpu().numpy()
    for s in range(b):
        r = accept_greedy_walk(base[s], tok[s], plan.parent, K)
        assert Lh[s] == r[0] and list(ph[s]) == list(r[1]) and list(ah[s]) == list(r[2])
        assert bh[s] == r[3]
    assert Lh[0] == K and Lh[1] == 9
    # compaction of the accepted paths (17 moves for sequence 0)
    nkv, d = 2, 64
    Pmax = P + T
    Kc = normal((b, nkv, Pmax, d), 779, 1.0, torch.bfloat16)
    Vc = normal((b, nkv, Pmax, d), 780, 1.0, torch.bfloat16)
    Kd, Vd = Kc.to(DEV), Vc.to(DEV)
    seq = torch.full((b,), P, **I32)
    M.medusa_kv_compact(Kd, Vd, seq, path, Lg)
    torch.cuda.synchronize()
    for s in range(b):
        Kn, Vn, nseq = kv_compact(Kc[s].float().numpy(), Vc[s].float().numpy(), P, ph[s], int(Lh[s]))
        assert int(seq[s]) == nseq
        assert np.array_equal(Kd[s].float().cpu().numpy(), Kn)
        assert np.array_equal(Vd[s].float().cpu().numpy(), Vn)
