"""The fused calls against the separate ones, bit for bit.

medusa_topk_tree must write exactly what medusa_topk followed by
medusa_build_tree writes, and medusa_accept_compact exactly what medusa_accept
followed by medusa_kv_compact writes (outputs, cache and seq_len).  Both paths
run from identical device inputs; the separate path is itself checked against
the oracle in test_gpu_stages / test_gpu_fullsize.
"""

import pytest
import torch

from speculative_decoding_heads_amd import configs as C
from speculative_decoding_heads_amd.step import VerifyStep, device_inputs
from speculative_decoding_heads_amd.synth import make_inputs
from tests.helpers import require_gpu, say

pytestmark = pytest.mark.gpu

SMALL = [
    C.TINY,
    # bf16, greedy, sparse tree, grouped heads
    C.Config("fused_bf16_greedy", 91, 3, 256, 3000, (4, 3, 2), 20, 4, 2, 64, 300, "bf16", "greedy"),
    # bf16, typical (the root and the next token are counter draws), long-ish tree
    C.Config("fused_bf16_typical", 92, 2, 384, 5000, (5, 4, 3, 2), 60, 6, 3, 64, 700, "bf16",
             "typical"),
    C.LLAMA7B_BS1,
    # rows * V >= 2^24: the verify GEMM leaves acceptance partials (ring kernel, greedy)
    C.Config("fused_parts_ring", 93, 8, 128, 40000, (4, 4, 4), 64, 2, 1, 64, 200, "bf16", "greedy"),
    # same with the tiled kernel (65 rows) and typical acceptance
    C.Config("fused_parts_tiled", 94, 1, 128, 260000, (4, 4, 4), 64, 2, 2, 64, 300, "bf16",
             "typical"),
    C.LLAMA7B_BS16,
]

OUTS = ("logits", "root", "idx", "val", "tokens", "pos", "parent", "depth", "anc", "O",
        "base_logits", "L", "path", "acc_tokens", "bonus")


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_fused_calls_match_separate_calls(cfg):
    say("fused vs separate", cfg.name)
    host = make_inputs(cfg)
    res = {}
    for fused in (False, True):
        x = device_inputs(cfg, host)
        st = VerifyStep(cfg)
        st.run(x, step=3, fused=fused)
        torch.cuda.synchronize()
        res[fused] = ({k: getattr(st, k).clone() for k in OUTS},
                      {k: x[k].clone() for k in ("Kc", "Vc", "seq_len")})
    (a, ca), (b, cb) = res[False], res[True]
    for k in OUTS:
        assert torch.equal(a[k], b[k]), k
    for k in ("Kc", "Vc", "seq_len"):
        assert torch.equal(ca[k], cb[k]), k
    # the rollback did run: seq_len = P + L + 1
    assert torch.equal(cb["seq_len"].cpu(), cfg.P + b["L"].cpu() + 1)


@pytest.mark.parametrize("rows,H,V", [(65, 256, 2000), (1040, 256, 3000), (5, 384, 31000),
                                      (122, 384, 5000), (11, 256, 4096),
                                      # the LDS-DMA weight stream (non-temporal weights in
                                      # the verify call, ordinary ones in medusa_heads)
                                      (65, 256, 32000), (5, 384, 32000), (80, 128, 262144)])
@pytest.mark.parametrize("mode", ["greedy", "typical"])
def test_verify_logits_match_heads(rows, H, V, mode):
    """medusa_verify_logits writes the same logits as medusa_heads (one kernel
    choice for both), whatever it leaves in its workspace."""
    from speculative_decoding_heads_amd import medusa as M
    from speculative_decoding_heads_amd.synth import normal
    say("verify logits", rows, H, V, mode)
    dt = torch.float32 if rows == 11 else torch.bfloat16
    x = normal((rows, H), rows + 7, 1.0, dt).to("cuda")
    LM = normal((V, H), rows + 8, 0.02, dt).to("cuda")
    a = torch.empty(rows, V, device="cuda")
    b = torch.empty(rows, V, device="cuda")
    M.medusa_heads(x, None, LM, a, include_base=1)
    md = M.TYPICAL if mode == "typical" else M.GREEDY
    ws = M.workspace(M.medusa_verify_workspace(rows, H, V, M.dtype_code(x), md))
    M.medusa_verify_logits(x, LM, b, md, 0.7, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("verify_mode,verify_temp", [("greedy", 1.0), ("typical", 0.9)])
def test_mismatched_verify_workspace_reads_the_logits(verify_mode, verify_temp):
    """Partials made for another call (greedy keys, or another temperature) are
    not used by a typical acceptance: it reads the logits instead and decides
    as the oracle does on them."""
    import numpy as np
    from oracle import accept_typical, counter_uniform, sample_tempered, tree_plan
    from speculative_decoding_heads_amd import medusa as M
    from speculative_decoding_heads_amd.synth import normal
    say("mismatched verify workspace", verify_mode, verify_temp)
    k, N, b, H, V = (4, 4, 4), 64, 8, 128, 40000
    plan = tree_plan(k, N)
    T, K = plan.T, len(k)
    rows = b * T
    assert rows * V >= 1 << 24          # the verify call keeps partials
    x = normal((rows, H), 501, 1.0, torch.bfloat16).to("cuda")
    LM = normal((V, H), 502, 0.4, torch.bfloat16).to("cuda")
    logits = torch.empty(rows, V, device="cuda")
    vmode = M.GREEDY if verify_mode == "greedy" else M.TYPICAL
    vws = M.workspace(M.medusa_verify_workspace(rows, H, V, M.BF16, vmode))
    M.medusa_verify_logits(x, LM, logits, vmode, verify_temp, vws)
    torch.cuda.synchronize()
    # children take ranked tokens of their parent's row, starting deeper in the
    # ranking for later sequences, so some paths stop early and some do not
    bl = logits.view(b, T, V).cpu().numpy()
    offs = [0, 1, 2, 4, 8, 16, 64, 1000]
    tokens = np.zeros((b, T), dtype=np.int32)
    for s in range(b):
        for p in range(T):
            kids = [c for c in range(1, T) if plan.parent[c] == p]
            if kids:
                order = np.argsort(-bl[s, p].astype(np.float64), kind="stable")
                tokens[s, kids] = order[[offs[s] + 3 * j for j in range(len(kids))]]
    tk = torch.from_numpy(tokens).to("cuda")
    par = torch.tensor(plan.parent, dtype=torch.int32, device="cuda")
    dep = torch.tensor(plan.depth, dtype=torch.int32, device="cuda")
    nkv, d, P = 1, 64, 10
    Kc = normal((b, nkv, P + T, d), 503, 1.0, torch.bfloat16).to("cuda")
    Vc = normal((b, nkv, P + T, d), 504, 1.0, torch.bfloat16).to("cuda")
    seq = torch.full((b,), P, dtype=torch.int32, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    L, path = torch.empty(b, **i32), torch.empty(b, K + 1, **i32)
    acc, bonus = torch.empty(b, K + 1, **i32), torch.empty(b, **i32)
    ws = M.workspace(M.medusa_accept_workspace(b, T))
    Tf = float(np.float32(0.7))
    M.medusa_accept_compact(logits.view(b, T, V), tk, par, dep, K, M.TYPICAL, Tf, 0.3, 0.09, 11,
                            3, L, path, acc, bonus, Kc, Vc, seq, ws, verify_ws=vws)
    torch.cuda.synchronize()
    Lh, ph, ah, bh = (t.cpu().numpy() for t in (L, path, acc, bonus))
    compared = 0
    for s in range(b):
        r = accept_typical(bl[s], tokens[s], plan.parent, plan.depth, K, Tf, np.float32(0.3),
                           np.float32(0.09), 11, 3, s)
        if np.min(r[4][1:]) < 1e-4:
            continue
        assert Lh[s] == r[0] and list(ph[s]) == list(r[1]) and list(ah[s]) == list(r[2])
        u = counter_uniform(11, 3, s, 1)
        want, cdf = sample_tempered(bl[s, r[1][r[0]]], Tf, u)
        if np.min(np.abs(cdf - u * cdf[-1])) / cdf[-1] > 1e-12:
            assert bh[s] == want
        compared += 1
    assert compared >= b - 1, compared
    # the decisions are not trivial on these logits: paths of several lengths
    assert len(set(Lh.tolist())) >= 3, Lh


@pytest.mark.parametrize("b,H,V,K,dt", [(1, 4096, 32000, 4, "bf16"), (16, 256, 3000, 4, "bf16"),
                                        (3, 384, 1000, 1, "bf16"), (1, 256, 4096, 3, "f32")])
def test_split_heads_match_medusa_heads(b, H, V, K, dt):
    """medusa_heads_hidden + medusa_lm_logits(reverse_k=1) write exactly what
    medusa_heads writes (u and logits); medusa_lm_logits(reverse_k=0) is the
    n_heads = 0 form."""
    from speculative_decoding_heads_amd import medusa as M
    from speculative_decoding_heads_amd.synth import normal
    say("split heads", b, H, V, K, dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    h = normal((b, H), 61 + b, 1.0, tdt).to("cuda")
    W = normal((K, H, H), 62 + b, 0.02, tdt).to("cuda")
    LM = normal((V, H), 63 + b, 0.02, tdt).to("cuda")
    u1 = torch.empty(b, K + 1, H, dtype=tdt, device="cuda")
    u2 = torch.empty_like(u1)
    l1 = torch.empty(b, K + 1, V, device="cuda")
    l2 = torch.empty_like(l1)
    M.medusa_heads(h, W, LM, l1, include_base=1, u_out=u1)
    M.medusa_heads_hidden(h, W, u2, include_base=1)
    M.medusa_lm_logits(u2, LM, l2, reverse_k=1)
    v1 = torch.empty(b * (K + 1), V, device="cuda")
    v2 = torch.empty_like(v1)
    M.medusa_heads(u1.view(-1, H), None, LM, v1, include_base=1)
    M.medusa_lm_logits(u1, LM, v2, reverse_k=0)
    torch.cuda.synchronize()
    assert torch.equal(u1, u2)
    assert torch.equal(l1, l2)
    assert torch.equal(v1, v2)


@pytest.mark.parametrize("mode", ["greedy", "typical"])
def test_weight_stream_partials_decide_as_the_logits(mode):
    """Acceptance partials written by the LDS-DMA weight-stream GEMM (68 verify
    rows over a 262144-entry vocabulary, past the 2^24 logits from which the
    verify call keeps partials) give the same acceptance as folding the logits
    rows (medusa_accept on the same logits), on a tree whose tokens are taken
    from the rows' own ranking so that paths of every length occur."""
    import numpy as np
    from oracle import tree_plan
    from speculative_decoding_heads_amd import medusa as M
    from speculative_decoding_heads_amd.synth import normal
    say("weight-stream partials", mode)
    k, b, H, V = (4, 3), 4, 256, 262144
    plan = tree_plan(k, None)
    T, K = plan.T, len(k)
    rows = b * T
    assert rows <= 80 and rows * V >= 1 << 24
    x = normal((rows, H), 611, 1.0, torch.bfloat16).to("cuda")
    LM = normal((V, H), 612, 0.4, torch.bfloat16).to("cuda")
    md = M.TYPICAL if mode == "typical" else M.GREEDY
    logits = torch.empty(rows, V, device="cuda")
    vws = M.workspace(M.medusa_verify_workspace(rows, H, V, M.BF16, md))
    Tf = float(np.float32(0.7))
    M.medusa_verify_logits(x, LM, logits, md, Tf, vws)
    ref = torch.empty(rows, V, device="cuda")
    M.medusa_lm_logits(x, LM, ref)
    torch.cuda.synchronize()
    assert torch.equal(logits, ref)
    bl = logits.view(b, T, V).cpu().numpy()
    tokens = np.zeros((b, T), dtype=np.int32)
    for s in range(b):
        for p in range(T):
            kids = [c for c in range(1, T) if plan.parent[c] == p]
            if kids:
                order = np.argsort(-bl[s, p].astype(np.float64), kind="stable")
                tokens[s, kids] = order[[s + 2 * j for j in range(len(kids))]]
    tk = torch.from_numpy(tokens).to("cuda")
    par = torch.tensor(plan.parent, dtype=torch.int32, device="cuda")
    dep = torch.tensor(plan.depth, dtype=torch.int32, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    outs = []
    for use_parts in (True, False):
        nkv, d, P = 1, 64, 10
        Kc = normal((b, nkv, P + T, d), 613, 1.0, torch.bfloat16).to("cuda")
        Vc = normal((b, nkv, P + T, d), 614, 1.0, torch.bfloat16).to("cuda")
        seq = torch.full((b,), P, **i32)
        L, path = torch.empty(b, **i32), torch.empty(b, K + 1, **i32)
        acc, bonus = torch.empty(b, K + 1, **i32), torch.empty(b, **i32)
        ws = M.workspace(M.medusa_accept_workspace(b, T))
        M.medusa_accept_compact(logits.view(b, T, V), tk, par, dep, K, md, Tf, 0.3, 0.09, 11, 3,
                                L, path, acc, bonus, Kc, Vc, seq, ws,
                                verify_ws=vws if use_parts else None)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (L, path, acc, bonus, Kc, Vc, seq)])
    for a_, b_ in zip(*outs):
        assert torch.equal(a_, b_)
    Ls = outs[0][0].tolist()
    if mode == "greedy":
        # sequence s offers rank s as the first child: only sequence 0 accepts
        assert Ls[0] == K and all(v == 0 for v in Ls[1:]), Ls
