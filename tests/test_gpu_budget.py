"""The tree budget on the GPU, against the oracle bit for bit:

  * medusa_topk_tree_tables on a tree planned from per-rank acceptance rates:
    shortlists and root as the oracle's stable top-k / argmax / counter
    sample, tree tables and tokens as the oracle's gather on that tree;
  * the same call on the fixed tree's tables equals medusa_topk_tree;
  * medusa_accept_tally against the oracle tally, over two batches added to
    the same counts, with out-of-range L rows skipped;
  * a loop of steps on a rates-planned tree, tallied after every step, equals
    the oracle tally of the steps' own L and paths.
"""

import numpy as np
import pytest
import torch

from oracle import (accept_tally, argmax_lowest, counter_uniform, plan_from_tables,
                    sample_tempered, topk_stable, tree_gather, tree_plan_rates)
from speculative_decoding_heads_amd import configs as C
from speculative_decoding_heads_amd import medusa as M
from speculative_decoding_heads_amd.step import VerifyLoop, device_inputs, loop_inputs
from speculative_decoding_heads_amd.synth import make_inputs
from tests.helpers import normal, require_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
I32 = dict(dtype=torch.int32, device=DEV)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _rates(k, seed):
    rng = np.random.default_rng(seed)
    q = np.zeros((len(k), 16))
    for d, s in enumerate(k):
        q[d, :s] = np.sort(rng.random(s))[::-1] * 0.8 ** d
    q[0, 1 % k[0]] = q[0, 0]            # a tie between two ranks of head 1
    return q


def _tree_outputs(b, T):
    W = (T + 63) // 64
    return (torch.empty(b, T, **I32), torch.empty(b, T, **I32), torch.empty(T, **I32),
            torch.empty(T, **I32), torch.empty(T, W, dtype=torch.int64, device=DEV))


def _check_tables(plan, parent, depth, anc):
    assert list(parent.cpu().numpy()) == list(plan.parent)
    assert list(depth.cpu().numpy()) == list(plan.depth)
    a = anc.cpu().numpy().view(np.uint64)
    for i in range(plan.T):
        for j in range(plan.T):
            assert bool((int(a[i, j // 64]) >> (j % 64)) & 1) == bool(plan.anc[i, j])


CASES = [((10,) * 4, 64, 3, 5000), ((3, 2, 2), 7, 2, 999), ((16, 16), 255, 1, 3000),
         ((4,), 0, 2, 100), ((2, 2, 1), None, 2, 4096)]


@pytest.mark.parametrize("k,N,b,V", CASES)
@pytest.mark.parametrize("mode", ["greedy", "typical", "given"])
def test_topk_tree_tables_matches_oracle(k, N, b, V, mode):
    say("topk_tree_tables", k, N, b, V, mode)
    K, kmax = len(k), max(k)
    par, dep, rk, _ = M.medusa_tree_plan_rates(k, N, _rates(k, len(k) + b))
    plan = plan_from_tables(k, par, rk)
    T = plan.T
    logits = normal((b, K + 1, V), 17 * b + V, 1.5, torch.float32)
    rng = np.random.default_rng(V)
    P = torch.from_numpy(rng.integers(0, 9000, size=b).astype(np.int32)).to(DEV)
    given = rng.integers(0, V, size=b).astype(np.int32)
    root = torch.from_numpy(given).to(DEV) if mode == "given" else torch.empty(b, **I32)
    idx = torch.empty(b, K, kmax, **I32)
    val = torch.empty(b, K, kmax, dtype=torch.float32, device=DEV)
    tokens, pos, parent, depth, anc = _tree_outputs(b, T)
    ws = M.workspace(M.medusa_topk_workspace(b, K, V, kmax))
    root_mode = {"greedy": M.GREEDY, "typical": M.TYPICAL, "given": M.ROOT_GIVEN}[mode]
    temp = float(np.float32(0.7))
    M.medusa_topk_tree_tables(logits.to(DEV), k, kmax, par, rk, root_mode, temp, 0x5EED, 5, P, root,
                              idx, val, tokens, pos, parent, depth, anc, ws)
    torch.cuda.synchronize()
    _check_tables(plan, parent, depth, anc)
    x = logits.numpy()
    r_gpu, i_gpu, v_gpu = root.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()
    for s in range(b):
        if mode == "greedy":
            assert r_gpu[s] == argmax_lowest(x[s, 0])
        elif mode == "given":
            assert r_gpu[s] == given[s]
        else:
            u = counter_uniform(0x5EED, 5, s, 0)
            want, c = sample_tempered(x[s, 0], temp, u)
            if np.min(np.abs(c - u * c[-1])) / c[-1] > 1e-12:
                assert r_gpu[s] == want
        for i in range(K):
            want = topk_stable(x[s, i + 1], k[i])
            assert list(i_gpu[s, i, : k[i]]) == list(want)
            assert np.array_equal(v_gpu[s, i, : k[i]], x[s, i + 1][want].astype(np.float32))
        tk, ps = tree_gather(plan, int(r_gpu[s]), i_gpu[s], int(P[s]))
        assert list(tokens[s].cpu().numpy()) == list(tk)
        assert list(pos[s].cpu().numpy()) == list(ps)


def test_topk_tree_tables_on_the_fixed_tree_equals_topk_tree():
    k, N, b, V = (10,) * 4, 64, 2, 32000
    K, kmax = len(k), max(k)
    par, _, rk = M.medusa_tree_plan(k, N)
    T = len(par)
    logits = normal((b, K + 1, V), 4242, 1.0, torch.float32).to(DEV)
    P = torch.tensor([100, 2000], **I32)
    ws = M.workspace(M.medusa_topk_workspace(b, K, V, kmax))
    outs = []
    for use_tables in (False, True):
        root = torch.empty(b, **I32)
        idx = torch.empty(b, K, kmax, **I32)
        val = torch.empty(b, K, kmax, dtype=torch.float32, device=DEV)
        tree = _tree_outputs(b, T)
        if use_tables:
            M.medusa_topk_tree_tables(logits, k, kmax, par, rk, M.GREEDY, 1.0, 1, 2, P, root, idx,
                                      val, *tree, ws)
        else:
            M.medusa_topk_tree(logits, k, kmax, N, 4, 5, M.GREEDY, 1.0, 1, 2, P, root, idx, val,
                               *tree, ws)
        torch.cuda.synchronize()
        outs.append([root, idx, val, *tree])
    for a, c in zip(*outs):
        assert torch.equal(a, c)


def _random_paths(plan, K, b, rng):
    children = {i: [] for i in range(plan.T)}
    for i in range(1, plan.T):
        children[int(plan.parent[i])].append(i)
    L = np.zeros(b, dtype=np.int32)
    path = np.full((b, K + 1), -1, dtype=np.int32)
    for s in range(b):
        node, d = 0, 0
        path[s, 0] = 0
        stop = rng.integers(0, K + 1)
        while d < stop and children[node]:
            node = int(rng.choice(children[node]))
            d += 1
            path[s, d] = node
        L[s] = d
    return L, path


def test_accept_tally_matches_oracle():
    k, N = (10,) * 4, 64
    K = len(k)
    par, _, rk, _ = M.medusa_tree_plan_rates(k, N, _rates(k, 9))
    plan = plan_from_tables(k, par, rk)
    rng = np.random.default_rng(31)
    acc = torch.zeros(K, 16, dtype=torch.int64, device=DEV)
    off = torch.zeros(K, 16, dtype=torch.int64, device=DEV)
    want_acc = np.zeros((K, 16), dtype=np.int64)
    want_off = np.zeros((K, 16), dtype=np.int64)
    for b in (50, 7):
        L, path = _random_paths(plan, K, b, rng)
        L[0], L[1] = -1, K + 1                 # out of range: skipped
        M.medusa_accept_tally(torch.from_numpy(L).to(DEV), torch.from_numpy(path).to(DEV), k, par,
                              rk, acc, off)
        a, o = accept_tally(plan, K, L, path)
        want_acc += a
        want_off += o
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), want_acc)
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert want_off.sum() > 0 and want_acc.sum() > 0


def test_loop_on_rates_tree_and_its_tally():
    cfg = C.Config("budget_loop", 98, 2, 384, 5000, (5, 4, 3), 40, 6, 3, 64, 200, "bf16", "typical")
    steps = 3
    par, _, rk, _ = M.medusa_tree_plan_rates(cfg.k, cfg.N, _rates(cfg.k, 3))
    plan = plan_from_tables(cfg.k, par, rk)
    host = make_inputs(cfg)
    x = device_inputs(cfg, host)
    cap = cfg.P + steps * (cfg.K + 1) + cfg.T
    for name in ("Kc", "Vc"):
        big = torch.zeros(cfg.b, cfg.nkv, cap, cfg.d, dtype=x[name].dtype, device=DEV)
        big[:, :, : cfg.P] = x[name][:, :, : cfg.P]
        x[name] = big
    Qs, Kn, Vn = loop_inputs(cfg, steps, seed_base=77)
    loop = VerifyLoop(cfg, plan=(par, rk))
    st = loop.step
    acc = torch.zeros(cfg.K, 16, dtype=torch.int64, device=DEV)
    off = torch.zeros(cfg.K, 16, dtype=torch.int64, device=DEV)
    rec = []

    def after(s):
        M.medusa_accept_tally(st.L, st.path, cfg.k, par, rk, acc, off)
        torch.cuda.synchronize()
        rec.append((st.L.cpu().numpy().copy(), st.path.cpu().numpy().copy(),
                    st.tokens.cpu().numpy().copy()))

    loop.run(x, Qs, Kn, Vn, after_step=after)
    torch.cuda.synchronize()
    _check_tables(plan, st.parent, st.depth, st.anc)
    want_acc = np.zeros((cfg.K, 16), dtype=np.int64)
    want_off = np.zeros((cfg.K, 16), dtype=np.int64)
    for L, path, _ in rec:
        a, o = accept_tally(plan, cfg.K, L, path)
        want_acc += a
        want_off += o
    assert np.array_equal(acc.cpu().numpy(), want_acc)
    assert np.array_equal(off.cpu().numpy(), want_off)
    assert want_off.sum() >= steps * cfg.b
