"""Stage-wise GPU parity at small sizes: every output element against the oracle.

Shapes span several tiles of each kernel and end in ragged tails; discrete
outputs must match bit for bit, floating outputs within the per-row relative
tolerance (2e-2 bf16, 1e-5 f32).  Discrete stages run the oracle on the GPU's
own upstream values (so both sides decide on the same float32 numbers).
"""

import numpy as np
import pytest
import torch

from oracle import (heads as o_heads, lm_project, topk_stable, argmax_lowest, tree_plan,
                    tree_gather, tree_attention, accept_greedy_walk, accept_greedy_parallel,
                    accept_typical, kv_compact, counter_uniform, sample_tempered, round_bf16)
from oracle.accept import typical_local
from oracle.attention import tree_attention_head
from speculative_decoding_heads_amd import medusa as M
from tests.helpers import (TOL_BF16, TOL_F32, assert_rows_close, np64, require_gpu, say,
                           normal)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


# ------------------------------------------------------------------ heads
HEAD_CASES = [
    # b, H, V, K, dtype   (comments: the head GEMM / the LM projection)
    (1, 128, 1000, 4, "bf16"),     # skinny 1-block; one 16-row block, ragged vocab tile
    (3, 256, 4093, 2, "bf16"),     # V % 4 != 0: scalar logit stores
    (17, 384, 2048, 1, "bf16"),    # N = H < 8192, 17 rows: 16-row skinny workgroups with
                                   # two row blocks, both operands by LDS DMA; 3 K-chunks
                                   # (odd: wave 0 takes the last); 34 LM rows
    (16, 256, 3000, 4, "bf16"),    # N = 1024, 16 rows: skinny, one row block; 80 LM rows
    (32, 256, 1000, 1, "bf16"),    # N = H, 32 rows: the last row count on skinny workgroups
    (33, 256, 1000, 1, "bf16"),    # N = H, 33 rows: the first on the tiled kernel
    (40, 256, 1000, 4, "bf16"),    # 200 LM rows: tiled kernel, ragged M and N tiles
    (3, 2048, 1000, 16, "bf16"),   # 32768 head rows: 8-wave LDS-DMA weight stream, rotated K walk
    (8, 8192, 1000, 5, "bf16"),    # 40960 x 8192 head rows: the 10-wave LDS-DMA weight stream
    (1, 4096, 1000, 4, "bf16"),    # the 7B batch-1 heads: skinny, weights by LDS DMA, X in registers
    (16, 4096, 1000, 4, "bf16"),   # 16 rows, K = 4096: the same kernel at its row limit
    (2, 512, 1000, 16, "bf16"),    # the same kernel with 4 K-chunks: waves 0 and 2 get none
    (1, 256, 4096, 3, "f32"),      # tiny fp32 workload shape
    (5, 100, 777, 2, "f32"),
]


@pytest.mark.parametrize("b,H,V,K,dt", HEAD_CASES)
def test_heads(b, H, V, K, dt):
    say("heads", b, H, V, K, dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    bf16 = dt == "bf16"
    seed = 1000 * b + H + V + K
    h = normal((b, H), seed, 1.0, tdt)
    W = normal((K, H, H), seed + 1, 0.02, tdt)
    LM = normal((V, H), seed + 2, 0.02, tdt)
    u = torch.empty(b, K + 1, H, dtype=tdt, device=DEV)
    logits = torch.empty(b, K + 1, V, dtype=torch.float32, device=DEV)
    M.medusa_heads(h.to(DEV), W.to(DEV), LM.to(DEV), logits, include_base=1, u_out=u)
    torch.cuda.synchronize()
    u_ref, lg_ref = o_heads(np64(h), np64(W), np64(LM), bf16)
    tol = TOL_BF16 if bf16 else TOL_F32
    assert np.array_equal(np64(u[:, 0]), np64(h))
    assert_rows_close(np64(u), u_ref, tol, "u")
    assert_rows_close(np64(logits), lg_ref, tol, "logits")
    # stage-wise: the projection of the GPU's own u, float32 accumulation bound
    lg_stage = lm_project(np64(u).reshape(-1, H), np64(LM)).reshape(b, K + 1, V)
    assert_rows_close(np64(logits), lg_stage, 2e-5 if bf16 else TOL_F32, "logits(stage)")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_zero_head_weights_reduce_to_base_head_bitwise(dt):
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    b, H, V, K = 2, 256, 1500, 4
    h = normal((b, H), 7, 1.0, tdt)
    LM = normal((V, H), 8, 0.02, tdt)
    W = torch.zeros(K, H, H, dtype=tdt)
    u = torch.empty(b, K + 1, H, dtype=tdt, device=DEV)
    logits = torch.empty(b, K + 1, V, dtype=torch.float32, device=DEV)
    M.medusa_heads(h.to(DEV), W.to(DEV), LM.to(DEV), logits, u_out=u)
    torch.cuda.synchronize()
    for i in range(1, K + 1):
        assert torch.equal(u[:, i], u[:, 0])
        assert torch.equal(logits[:, i], logits[:, 0])
    ref = lm_project(np64(h), np64(LM))
    assert_rows_close(np64(logits[:, 0]), ref, TOL_BF16 if dt == "bf16" else TOL_F32, "base")


@pytest.mark.parametrize("b,H,V", [(1, 2048, 3000), (1, 1024, 32000), (3, 1536, 32003)])
def test_head_rows_and_base_rows_differ_only_in_summation_order(b, H, V):
    """With n_heads > 0 the LM projection walks K backwards (the n_heads = 0
    call forwards): slot 0 of the head call and the base-only call project the
    same x through the same bf16 products, summed in another order."""
    K = 4
    h = normal((b, H), 31 * b + H, 1.0, torch.bfloat16)
    W = normal((K, H, H), 32 * b + H, 0.02, torch.bfloat16)
    LM = normal((V, H), 33 * b + H, 0.02, torch.bfloat16)
    logits = torch.empty(b, K + 1, V, dtype=torch.float32, device=DEV)
    base = torch.empty(b, V, dtype=torch.float32, device=DEV)
    u = torch.empty(b, K + 1, H, dtype=torch.bfloat16, device=DEV)
    hd, LMd = h.to(DEV), LM.to(DEV)
    M.medusa_heads(hd, W.to(DEV), LMd, logits, include_base=1, u_out=u)
    M.medusa_heads(hd, None, LMd, base, include_base=1)
    torch.cuda.synchronize()
    a, c = np64(logits[:, 0]), np64(base)
    assert_rows_close(a, c, 2e-6, "slot 0 vs base-only")
    assert_rows_close(c, lm_project(np64(h), np64(LM)), 2e-5, "base-only")


@pytest.mark.parametrize("rows,H,V", [(65, 256, 2000), (1040, 256, 2000), (11, 256, 4096),
                                       (2080, 384, 1000), (300, 128, 777), (97, 512, 300),
                                       (5, 384, 31000), (65, 256, 30977), (16, 640, 33000),
                                       (80, 128, 30720), (5, 256, 40000), (65, 128, 50000),
                                       (16, 256, 60000), (161, 128, 40001),
                                       (1040, 384, 3333), (97, 256, 32000), (129, 384, 5000),
                                       (150, 256, 31000), (160, 128, 128256),
                                       # one ragged shape per remaining ring-GEMM tile:
                                       # 160x320, 192x256, 192x320, 224x256, 224x320,
                                       # 256x256, 256x320 (rows x weight rows)
                                       (257, 256, 40001), (321, 384, 32000), (321, 256, 40001),
                                       (385, 384, 32000), (385, 128, 40001), (449, 256, 32000),
                                       (449, 128, 40001)])
def test_verify_rows_projection(rows, H, V):
    dt = torch.float32 if rows == 11 else torch.bfloat16
    x = normal((rows, H), rows, 1.0, dt)
    LM = normal((V, H), rows + 1, 0.02, dt)
    out = torch.empty(rows, V, dtype=torch.float32, device=DEV)
    M.medusa_heads(x.to(DEV), None, LM.to(DEV), out, include_base=1)
    torch.cuda.synchronize()
    ref = lm_project(np64(x), np64(LM))
    assert_rows_close(np64(out), ref, 2e-5 if dt == torch.bfloat16 else TOL_F32, "verify rows")


@pytest.mark.parametrize("rows,H,V", [(1, 4096, 32000), (5, 4096, 32000), (17, 256, 32768),
                                      (33, 512, 32000), (48, 8192, 32000), (65, 4096, 32000),
                                      (80, 256, 128256)])
def test_weight_stream_logits_both_walks(rows, H, V):
    """The LDS-DMA weight-stream GEMM (at most 80 rows, vocabulary a multiple
    of 128 and at least 30720): forward and backward K walks, and the verify
    call's non-temporal weight reads, against the oracle's projection."""
    say("weight stream", rows, H, V)
    x = normal((rows, H), 7 * rows + 1, 1.0, torch.bfloat16)
    LM = normal((V, H), 7 * rows + 2, 0.02, torch.bfloat16)
    xd, LMd = x.to(DEV), LM.to(DEV)
    ref = lm_project(np64(x), np64(LM))
    ws = M.workspace(M.medusa_verify_workspace(rows, H, V, M.BF16, M.GREEDY))
    outs = []
    for rev in (0, 1, None):
        out = torch.full((rows, V), float("nan"), dtype=torch.float32, device=DEV)
        if rev is None:
            M.medusa_verify_logits(xd, LMd, out, M.GREEDY, 1.0, ws)
        else:
            M.medusa_lm_logits(xd, LMd, out, reverse_k=rev)
        torch.cuda.synchronize()
        assert_rows_close(np64(out), ref, 2e-5, f"logits rev={rev}")
        outs.append(out)
    assert torch.equal(outs[0], outs[2])      # the cache hint changes no value


# ------------------------------------------------------------------ top-k
def _topk_run(logits, k, kmax, mode, temperature=0.7, seed=5, step=3):
    b, K1, V = logits.shape
    K = K1 - 1
    root = torch.empty(b, dtype=torch.int32, device=DEV)
    idx = torch.empty(b, K, kmax, dtype=torch.int32, device=DEV)
    val = torch.empty(b, K, kmax, dtype=torch.float32, device=DEV)
    ws = M.workspace(M.medusa_topk_workspace(b, K, V, kmax))
    M.medusa_topk(logits.to(DEV), k, kmax, mode, temperature, seed, step, root, idx, val, ws)
    torch.cuda.synchronize()
    return root.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()


@pytest.mark.parametrize("b,K,V,k", [(1, 4, 32000, (10, 10, 10, 10)), (3, 3, 4093, (16, 1, 7)),
                                     (2, 2, 10000, (5, 3)), (4, 1, 20, (16,)),
                                     (1, 5, 9000, (4, 4, 4, 4, 4))])
def test_topk_greedy_exact(b, K, V, k):
    say("topk", b, K, V, k)
    logits = normal((b, K + 1, V), b * V + K, 1.0, torch.float32)
    kmax = max(k)
    root, idx, val = _topk_run(logits, k, kmax, M.GREEDY)
    x = logits.numpy()
    for s in range(b):
        assert root[s] == argmax_lowest(x[s, 0])
        for i in range(K):
            want = topk_stable(x[s, i + 1], k[i])
            assert list(idx[s, i, : k[i]]) == list(want)
            assert np.array_equal(val[s, i, : k[i]], x[s, i + 1][want].astype(np.float32))
            assert all(idx[s, i, k[i]:] == -1) and np.all(np.isneginf(val[s, i, k[i]:]))


def test_topk_ties_signed_zero_and_small_vocab():
    b, K, V = 2, 3, 5000
    rng = np.random.default_rng(3)
    x = rng.integers(-2, 3, size=(b, K + 1, V)).astype(np.float32)   # massive ties
    x[0, 1, 100] = -0.0
    x[0, 1, 50] = 0.0
    x[1, 2, :] = 0.0
    x[1, 2, 4000:] = -0.0
    root, idx, val = _topk_run(torch.from_numpy(x), (16, 16, 16), 16, M.GREEDY)
    for s in range(b):
        assert root[s] == argmax_lowest(x[s, 0])
        for i in range(K):
            assert list(idx[s, i]) == list(topk_stable(x[s, i + 1], 16))


def test_topk_typical_root_is_counter_sample():
    b, K, V = 6, 2, 3001
    logits = normal((b, K + 1, V), 99, 2.0, torch.float32)
    T = float(np.float32(0.7))
    root, idx, _ = _topk_run(logits, (3, 3), 3, M.TYPICAL, temperature=T, seed=0x5EED, step=11)
    x = logits.numpy()
    for s in range(b):
        u = counter_uniform(0x5EED, 11, s, 0)
        want, c = sample_tempered(x[s, 0], T, u)
        margin = np.min(np.abs(c - u * c[-1])) / c[-1]
        if margin > 1e-12:
            assert root[s] == want
        assert list(idx[s, 0]) == list(topk_stable(x[s, 1], 3))


@pytest.mark.parametrize("V,scale", [(1, 1.0), (7, 3.0), (63, 1.0), (64, 2.0), (65, 0.5),
                                     (100, 30.0), (4097, 1.0), (32000, 0.05), (128256, 4.0)])
def test_typical_root_samples_across_vocab_sizes(V, scale):
    """The sampler cuts a row into 64 slices (empty ones when V < 64): many
    draws, flat to peaked rows, against the serial float64 rule."""
    b = 48
    logits = normal((b, 2, V), V + 5, scale, torch.float32)
    T = float(np.float32(0.7))
    root, _, _ = _topk_run(logits, (1,), 1, M.TYPICAL, temperature=T, seed=0xABC, step=V)
    x = logits.numpy()
    compared = 0
    for s in range(b):
        u = counter_uniform(0xABC, V, s, 0)
        want, c = sample_tempered(x[s, 0], T, u)
        if np.min(np.abs(c - u * c[-1])) / c[-1] > 1e-12:
            assert root[s] == want, (s, int(root[s]), want)
            compared += 1
    assert compared >= b - 2


# ------------------------------------------------------------------ tree
@pytest.mark.parametrize("k,N,b", [((2, 2, 1), None, 1), ((10,) * 4, 64, 3), ((10,) * 5, 128, 2),
                                   ((3, 2), 5, 1), ((16, 16), 255, 2), ((4,), 0, 2)])
def test_build_tree_exact(k, N, b):
    K, kmax = len(k), max(k)
    rng = np.random.default_rng(len(k) * 7 + b)
    idx = np.full((b, K, kmax), -1, dtype=np.int32)
    for s in range(b):
        for i in range(K):
            idx[s, i, : k[i]] = rng.choice(50000, size=k[i], replace=False)
    root = rng.integers(0, 50000, size=b).astype(np.int32)
    P = rng.integers(0, 5000, size=b).astype(np.int32)
    plan = tree_plan(k, N)
    T = plan.T
    W = (T + 63) // 64
    d = dict(dtype=torch.int32, device=DEV)
    tokens, pos = torch.empty(b, T, **d), torch.empty(b, T, **d)
    parent, depth = torch.empty(T, **d), torch.empty(T, **d)
    anc = torch.empty(T, W, dtype=torch.int64, device=DEV)
    M.medusa_build_tree(k, N, 4, 5, torch.from_numpy(root).to(DEV), torch.from_numpy(idx).to(DEV),
                        torch.from_numpy(P).to(DEV), tokens, pos, parent, depth, anc)
    torch.cuda.synchronize()
    assert list(parent.cpu().numpy()) == list(plan.parent)
    assert list(depth.cpu().numpy()) == list(plan.depth)
    a = anc.cpu().numpy().view(np.uint64)
    for i in range(T):
        for j in range(T):
            assert bool((int(a[i, j // 64]) >> (j % 64)) & 1) == bool(plan.anc[i, j])
    for s in range(b):
        tk, ps = tree_gather(plan, int(root[s]), idx[s], int(P[s]))
        assert list(tokens[s].cpu().numpy()) == list(tk)
        assert list(pos[s].cpu().numpy()) == list(ps)


# ------------------------------------------------------------------ attention
ATTN_CASES = [
    # b, k, N, nq, nkv, d, P, dtype
    (1, (2, 2, 1), None, 4, 4, 64, 128, "f32"),       # tiny workload shape
    (2, (3, 2), 5, 4, 2, 32, 77, "f32"),
    (1, (10,) * 4, 64, 4, 4, 128, 300, "bf16"),       # 65 rows per kv head, split keys
    (2, (10,) * 4, 64, 8, 2, 128, 1000, "bf16"),      # GQA 4, 260 rows, ragged P
    (1, (10,) * 5, 128, 8, 1, 128, 200, "bf16"),      # 129 nodes x 8 heads, 3 anc words
    (3, (2, 2), None, 2, 2, 64, 0, "bf16"),           # no prefix: tree only
    (2, (16, 15), 255, 2, 1, 128, 64, "bf16"),        # 256 nodes: 4 anc words
    (1, (1,), 0, 2, 2, 128, 5000, "bf16"),            # root only, long prefix
    (1, (10,) * 4, 64, 6, 2, 128, 700, "bf16"),       # GQA 3, 195 rows: 4 waves x 4 blocks
    (1, (10,) * 4, 64, 4, 2, 64, 300, "bf16"),        # d 64, 130 rows: 4 waves x 3 blocks
    (2, (10,) * 4, 64, 16, 2, 64, 500, "bf16"),       # d 64, 520 rows: 4 waves x 6 blocks, 2 groups
]


def _attn_inputs(b, T, nq, nkv, d, P, dt, seed, extra=5):
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    Pmax = P + T + extra
    Q = normal((b, T, nq, d), seed, 1.0, tdt)
    Kc = normal((b, nkv, Pmax, d), seed + 1, 1.0, tdt)
    Vc = normal((b, nkv, Pmax, d), seed + 2, 1.0, tdt)
    return Q, Kc, Vc, Pmax


def _anc_words(plan):
    T = plan.T
    W = (T + 63) // 64
    a = np.zeros((T, W), dtype=np.uint64)
    for i in range(T):
        for j in range(T):
            if plan.anc[i, j]:
                a[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return torch.from_numpy(a.view(np.int64))


@pytest.mark.parametrize("b,k,N,nq,nkv,d,P,dt", ATTN_CASES)
def test_tree_attention(b, k, N, nq, nkv, d, P, dt):
    say("attn", b, k, N, nq, nkv, d, P, dt)
    plan = tree_plan(k, N)
    T = plan.T
    Q, Kc, Vc, Pmax = _attn_inputs(b, T, nq, nkv, d, P, dt, seed=T * 31 + P)
    Pv = np.array([P - (s % 2) * min(P, 3) for s in range(b)], dtype=np.int32)  # ragged prefixes
    seq = torch.from_numpy(Pv).to(DEV)
    O = torch.empty(b, T, nq * d, dtype=Q.dtype, device=DEV)
    dtc = M.BF16 if dt == "bf16" else M.F32
    ws = M.workspace(M.medusa_tree_attn_workspace(b, T, nq, nkv, d, Pmax, dtc))
    M.medusa_tree_attn(Q.to(DEV), Kc.to(DEV), Vc.to(DEV), seq, _anc_words(plan).to(DEV), O, ws=ws)
    torch.cuda.synchronize()
    ref = tree_attention(np64(Q), np64(Kc), np64(Vc), Pv, plan.anc, bf16=(dt == "bf16"))
    got = np64(O).reshape(b, T, nq, d)
    assert_rows_close(got, ref.reshape(b, T, nq, d), TOL_BF16 if dt == "bf16" else TOL_F32, "O")


# Shapes that put the attention plan on its larger row groups (the cost model
# picks them only with enough (sequence, kv head) pairs to fill the CUs) and
# on the 2-deep K/V ring (two workgroups per CU):
# b, k, N, nq, nkv, d, P, and the plan the model gives (blocks per group,
# groups, key partitions) for the reader; the test checks the split decision
# through the workspace size and every node of one q head per (sequence, kv
# head) against the oracle.
ATTN_PLAN_CASES = [
    # blocks per group x groups (last group), key partitions, ring depth
    (12, (6, 5), None, 64, 8, 128, 30, True),          # 4 x 5 (3), whole keys, 2-deep
    (2, (10,) * 5, 128, 8, 8, 128, 2000, False),       # 3 x 3, 5 partitions, 2-deep
    (16, (10,) * 4, 64, 32, 32, 128, 300, True),       # 5 x 1, whole keys, 2-deep
    (4, (1,), 0, 32, 32, 128, 2043, False),            # 1 x 1, 2 partitions, 2-deep
    (6, (4, 3, 2), 20, 256, 32, 128, 30, True),        # 11 x 1 (2 blocks per wave), 4-deep
    (3, (4, 3, 2), 20, 64, 8, 128, 4000, False),       # 11 x 1, 9 partitions
    (4, (10,) * 4, 64, 256, 32, 128, 30, True),        # 17 x 2 (16; 3 blocks per wave)
    (3, (6, 5), None, 128, 16, 128, 4000, False),      # 19 x 1, 5 partitions
    (16, (10,) * 4, 64, 64, 8, 64, 30, True),          # d 64: 11 x 3
    (8, (10,) * 4, 64, 32, 8, 64, 2000, False),        # d 64: 9 x 2 (8), 4 partitions
    (2, (10,) * 4, 64, 256, 32, 64, 4000, False),      # d 64: 17 x 2 (16), 4 partitions
]


@pytest.mark.parametrize("b,k,N,nq,nkv,d,P,whole", ATTN_PLAN_CASES)
def test_tree_attention_row_groups(b, k, N, nq, nkv, d, P, whole):
    say("attn plan", b, k, N, nq, nkv, d, P)
    plan = tree_plan(k, N)
    T = plan.T
    G = nq // nkv
    Q, Kc, Vc, Pmax = _attn_inputs(b, T, nq, nkv, d, P, "bf16", seed=T * 17 + P + nq)
    ws_bytes = M.medusa_tree_attn_workspace(b, T, nq, nkv, d, Pmax, M.BF16)
    assert (ws_bytes == 0) == whole        # keys split <=> partials in the workspace
    Pv = np.array([P - (s % 2) * min(P, 3) for s in range(b)], dtype=np.int32)
    O = torch.empty(b, T, nq * d, dtype=Q.dtype, device=DEV)
    M.medusa_tree_attn(Q.to(DEV), Kc.to(DEV), Vc.to(DEV), torch.from_numpy(Pv).to(DEV),
                       _anc_words(plan).to(DEV), O, ws=M.workspace(ws_bytes))
    torch.cuda.synchronize()
    got = np64(O).reshape(b, T, nq, d)
    scale = 1.0 / np.sqrt(d)
    for s in range(b):
        for g in range(nkv):
            hq = g * G + (s + g) % G
            ref = tree_attention_head(np64(Q[s, :, hq]), np64(Kc[s, g]), np64(Vc[s, g]),
                                      int(Pv[s]), plan.anc, scale)
            assert_rows_close(got[s, :, hq], ref, TOL_BF16, f"O seq {s} kv head {g} q head {hq}")


def test_attention_invalid_seq_len_gives_nan_rows():
    plan = tree_plan((2, 2), None)
    T = plan.T
    Q, Kc, Vc, Pmax = _attn_inputs(2, T, 4, 4, 128, 100, "bf16", 5)
    seq = torch.tensor([100, Pmax], dtype=torch.int32, device=DEV)      # second: P + T > Pmax
    O = torch.empty(2, T, 4 * 128, dtype=torch.bfloat16, device=DEV)
    ws = M.workspace(M.medusa_tree_attn_workspace(2, T, 4, 4, 128, Pmax, M.BF16))
    M.medusa_tree_attn(Q.to(DEV), Kc.to(DEV), Vc.to(DEV), seq, _anc_words(plan).to(DEV), O, ws=ws)
    torch.cuda.synchronize()
    assert torch.isnan(O[1].float()).all()
    assert torch.isfinite(O[0].float()).all()


# ------------------------------------------------------------------ acceptance
def _plant(plan, V, rng, plant_p, scale=1.0):
    T = plan.T
    tokens = np.zeros(T, dtype=np.int32)
    tokens[0] = rng.integers(V)
    for p in range(T):
        kids = [c for c in range(1, T) if plan.parent[c] == p]
        if kids:
            tokens[kids] = rng.choice(V, size=len(kids), replace=False)
    x = rng.standard_normal((T, V)).astype(np.float32) * scale
    for c in range(1, T):
        if rng.random() < plant_p:
            p = plan.parent[c]
            x[p, tokens[c]] = x[p].max() + 1.0
    return tokens, x


def _accept_run(x, tokens, plan, K, mode, T_=0.7, eps=0.3, delta=0.09, seed=9, step=4):
    b, T, V = x.shape
    d = dict(dtype=torch.int32, device=DEV)
    L, path = torch.empty(b, **d), torch.empty(b, K + 1, **d)
    acc, bonus = torch.empty(b, K + 1, **d), torch.empty(b, **d)
    ws = M.workspace(M.medusa_accept_workspace(b, T))
    M.medusa_accept(torch.from_numpy(x).to(DEV), torch.from_numpy(tokens).to(DEV),
                    torch.tensor(plan.parent, dtype=torch.int32, device=DEV),
                    torch.tensor(plan.depth, dtype=torch.int32, device=DEV), K, mode, T_, eps, delta,
                    seed, step, L, path, acc, bonus, ws)
    torch.cuda.synchronize()
    return L.cpu().numpy(), path.cpu().numpy(), acc.cpu().numpy(), bonus.cpu().numpy()


@pytest.mark.parametrize("k,N,V,plant", [((10,) * 4, 64, 32000, 0.5), ((10,) * 5, 128, 3001, 0.7),
                                         ((2, 2, 1), None, 4096, 0.9), ((3, 3), None, 50, 0.0),
                                         ((16, 15), 255, 1000, 0.4)])
def test_accept_greedy_exact(k, N, V, plant):
    plan = tree_plan(k, N)
    K = len(k)
    rng = np.random.default_rng(V + K)
    b = 4
    toks, xs = zip(*[_plant(plan, V, rng, plant) for _ in range(b)])
    tokens, x = np.stack(toks), np.stack(xs)
    L, path, acc, bonus = _accept_run(x, tokens, plan, K, M.GREEDY)
    for s in range(b):
        w = accept_greedy_walk(x[s], tokens[s], plan.parent, K)
        p = accept_greedy_parallel(x[s], tokens[s], plan.parent, plan.depth, K)
        assert w[0] == p[0]
        assert L[s] == w[0], (s, L[s], w[0])
        assert list(path[s]) == list(w[1]) and list(acc[s]) == list(w[2]) and bonus[s] == w[3]


@pytest.mark.parametrize("k,N,V,scale", [((10,) * 4, 64, 32000, 1.0), ((10,) * 4, 64, 5000, 25.0),
                                         ((4, 4, 4), 40, 3001, 8.0), ((2, 2, 1), None, 100, 3.0)])
def test_accept_typical_exact(k, N, V, scale):
    plan = tree_plan(k, N)
    K = len(k)
    rng = np.random.default_rng(V + 3)
    b = 5
    Tf = float(np.float32(0.7))
    toks, xs = zip(*[_plant(plan, V, rng, 0.5, scale) for _ in range(b)])
    tokens, x = np.stack(toks), np.stack(xs)
    L, path, acc, bonus = _accept_run(x, tokens, plan, K, M.TYPICAL, T_=Tf, seed=77, step=2)
    compared = bonus_compared = 0
    for s in range(b):
        r = accept_typical(x[s], tokens[s], plan.parent, plan.depth, K, Tf, 0.3, 0.09, 77, 2, s)
        guarded = np.min(r[4][1:]) < 1e-4
        if not guarded:
            assert L[s] == r[0] and list(path[s]) == list(r[1]) and list(acc[s]) == list(r[2])
            compared += 1
            best = r[1][r[0]]
            u = counter_uniform(77, 2, s, 1)
            want, c = sample_tempered(x[s, best], Tf, u)
            if np.min(np.abs(c - u * c[-1])) / c[-1] > 1e-12:
                assert bonus[s] == want == r[3]
                bonus_compared += 1
    # on these seeds no decision or draw lies within the guard bands (the
    # oracle alone decides that), so every sequence must have been compared
    assert compared == b and bonus_compared == b, (compared, bonus_compared)


def test_accept_typical_eps_branch():
    # eps < delta: the threshold is eps for peaked parents
    plan = tree_plan((3, 3), None)
    rng = np.random.default_rng(4)
    tokens, x = _plant(plan, 200, rng, 0.6, 6.0)
    x, tokens = x[None], tokens[None]
    L, path, acc, bonus = _accept_run(x, tokens, plan, 2, M.TYPICAL, T_=1.0, eps=0.02, delta=0.5,
                                      seed=3, step=0)
    r = accept_typical(x[0], tokens[0], plan.parent, plan.depth, 2, 1.0, 0.02, 0.5, 3, 0, 0)
    assert np.min(r[4][1:]) > 1e-4
    assert L[0] == r[0] and list(path[0]) == list(r[1])


# ------------------------------------------------------------------ compaction
@pytest.mark.parametrize("dt,nkv,d", [("bf16", 4, 128), ("f32", 2, 64), ("bf16", 3, 64)])
def test_kv_compact_exact(dt, nkv, d):
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    b, K, P, T = 4, 4, 37, 30
    Pmax = P + T + 3
    Kc = normal((b, nkv, Pmax, d), 5, 1.0, tdt)
    Vc = normal((b, nkv, Pmax, d), 6, 1.0, tdt)
    paths = np.array([[0, 2, 5, 9, 20], [0, 1, 2, 3, 4], [0, -1, -1, -1, -1], [0, 3, 8, -1, -1]],
                     dtype=np.int32)
    Ls = np.array([4, 4, 0, 2], dtype=np.int32)
    seq = torch.full((b,), P, dtype=torch.int32, device=DEV)
    Kd, Vd = Kc.to(DEV), Vc.to(DEV)
    M.medusa_kv_compact(Kd, Vd, seq, torch.from_numpy(paths).to(DEV), torch.from_numpy(Ls).to(DEV))
    torch.cuda.synchronize()
    for s in range(b):
        Kn, Vn, n = kv_compact(Kc[s].float().numpy(), Vc[s].float().numpy(), P, paths[s], int(Ls[s]))
        assert int(seq[s]) == n
        assert np.array_equal(Kd[s].float().cpu().numpy(), Kn)
        assert np.array_equal(Vd[s].float().cpu().numpy(), Vn)


def test_kv_compact_long_paths():
    """Paths of up to 17 nodes (K = 16): several groups of moves per column."""
    tdt = torch.bfloat16
    b, K, nkv, d, P, T = 3, 16, 2, 64, 50, 40
    Pmax = P + T
    Kc = normal((b, nkv, Pmax, d), 15, 1.0, tdt)
    Vc = normal((b, nkv, Pmax, d), 16, 1.0, tdt)
    full = [0, 1, 3, 4, 6, 8, 9, 11, 14, 15, 17, 20, 22, 25, 28, 31, 39]
    nine = [0, 2, 4, 6, 8, 10, 12, 14, 16, 18] + [-1] * 7
    paths = np.array([full, nine, [0] + [-1] * 16], dtype=np.int32)
    Ls = np.array([16, 9, 0], dtype=np.int32)
    seq = torch.full((b,), P, dtype=torch.int32, device=DEV)
    Kd, Vd = Kc.to(DEV), Vc.to(DEV)
    M.medusa_kv_compact(Kd, Vd, seq, torch.from_numpy(paths).to(DEV), torch.from_numpy(Ls).to(DEV))
    torch.cuda.synchronize()
    for s in range(b):
        Kn, Vn, n = kv_compact(Kc[s].float().numpy(), Vc[s].float().numpy(), P, paths[s], int(Ls[s]))
        assert int(seq[s]) == n
        assert np.array_equal(Kd[s].float().cpu().numpy(), Kn)
        assert np.array_equal(Vd[s].float().cpu().numpy(), Vn)
