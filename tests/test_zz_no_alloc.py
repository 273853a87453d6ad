"""medusa_tree_attn_noalloc against medusa_tree_attn, through the C ABI.

The no-allocation call keeps the split-KV partials in the library's static
device scratch instead of a caller workspace; it must write exactly what
medusa_tree_attn writes with its own workspace.  Two calls in a row share
the scratch, the second with a smaller input; a shape whose partials exceed
the scratch is refused before anything is launched.
"""

import numpy as np
import pytest
import torch

from oracle import tree_plan
from speculative_decoding_heads_amd import medusa as M
from speculative_decoding_heads_amd.synth import normal
from tests.helpers import require_gpu, say

pytestmark = pytest.mark.gpu


def _case(b, k, N, nq, nkv, d, P, seed):
    plan = tree_plan(k, N)
    T = plan.T
    words = (T + 63) // 64
    anc = np.zeros((T, words), dtype=np.uint64)
    for i in range(T):
        for j in range(T):
            if plan.anc[i][j]:
                anc[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    Pmax = P + T
    x = dict(
        Q=normal((b, T, nq, d), seed, 1.0, torch.bfloat16).to("cuda"),
        Kc=normal((b, nkv, Pmax, d), seed + 1, 1.0, torch.bfloat16).to("cuda"),
        Vc=normal((b, nkv, Pmax, d), seed + 2, 1.0, torch.bfloat16).to("cuda"),
        seq_len=torch.full((b,), P, dtype=torch.int32, device="cuda"),
        anc=torch.from_numpy(anc.view(np.int64)).to("cuda"),
    )
    return x, (b, T, nq, nkv, d, Pmax)


def _reference(x, shape):
    b, T, nq, nkv, d, Pmax = shape
    ws_bytes = M.medusa_tree_attn_workspace(b, T, nq, nkv, d, Pmax, M.BF16)
    O = torch.empty(b, T, nq * d, dtype=torch.bfloat16, device="cuda")
    M.medusa_tree_attn(x["Q"], x["Kc"], x["Vc"], x["seq_len"], x["anc"], O,
                       ws=M.workspace(ws_bytes))
    return O, ws_bytes


def test_noalloc_attention_matches_the_workspace_call():
    require_gpu()
    limit = 16 << 20
    # a 7B-shape batch-1 step (64-candidate tree, 32 heads, prefix 2048), then
    # a smaller grouped-query input; both split the keys, so both use the scratch
    big, sb = _case(1, (10, 10, 10, 10), 64, 32, 32, 128, 2048, 700)
    small, ss = _case(2, (4, 3, 2), 20, 8, 2, 64, 700, 710)
    want_big, ws_big = _reference(big, sb)
    want_small, ws_small = _reference(small, ss)
    say("noalloc attention: partials", ws_big, "and", ws_small, "bytes")
    assert 0 < ws_small < ws_big <= limit
    got_big = torch.full_like(want_big, float("nan"))
    got_small = torch.full_like(want_small, float("nan"))
    M.medusa_tree_attn_noalloc(big["Q"], big["Kc"], big["Vc"], big["seq_len"], big["anc"],
                               got_big)
    torch.cuda.synchronize()
    assert torch.equal(got_big, want_big)
    M.medusa_tree_attn_noalloc(small["Q"], small["Kc"], small["Vc"], small["seq_len"],
                               small["anc"], got_small)
    torch.cuda.synchronize()
    assert torch.equal(got_small, want_small)
    # and once more on the larger input, after the smaller call left its partials
    got_big.fill_(float("nan"))
    M.medusa_tree_attn_noalloc(big["Q"], big["Kc"], big["Vc"], big["seq_len"], big["anc"],
                               got_big)
    torch.cuda.synchronize()
    assert torch.equal(got_big, want_big)


def test_noalloc_attention_refuses_partials_beyond_the_scratch():
    require_gpu()
    # the 70B-layer shape at batch 1 (129 nodes x 8 grouped heads, prefix
    # 8192) splits its keys five ways: about 21 MB of partials
    x, shape = _case(1, (10,) * 5, 128, 64, 8, 128, 8192, 720)
    b, T, nq, nkv, d, Pmax = shape
    assert M.medusa_tree_attn_workspace(b, T, nq, nkv, d, Pmax, M.BF16) > 16 << 20
    O = torch.zeros(b, T, nq * d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MedusaError) as e:
        M.medusa_tree_attn_noalloc(x["Q"], x["Kc"], x["Vc"], x["seq_len"], x["anc"], O)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert bool((O == 0).all())
