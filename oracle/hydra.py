"""Hydra-style sequentially dependent draft heads (oracle; test infrastructure
only).

zackli.ai "Speculative Decoding Deep Dive II: Medusa, MTP", section "Medusa":
the Medusa heads see only h_t and never the token just drafted, so their
accuracy falls with the offset; Hydra feeds that token to the later heads
(better drafts, less parallelism).  aicassindra.com "Medusa deep dive", "The
heads are residual blocks, not linear layers": a head is y + SiLU(W y)
followed by the shared LM projection.

Reading taken (the pages give Hydra one sentence), the same as the library's:
  * head d (1..K) takes y = h + e(x) in place of h, where e is the base
    model's input embedding table [V, H] and x the token one position earlier
    on the candidate's path: the root for head 1, the depth-(d-1) token for
    head d;
  * in bf16 mode y is rounded to bf16 once, then u = bf16(y + SiLU(W_d y)) as
    for the Medusa heads, and the logits are LM u unrounded;
  * every node of depth d-1 gets its own head-d logits and top-k_d
    (descending, ties to the lower index); node (r_1, ..., r_d) of the tree
    plan takes rank r_d of its parent's shortlist;
  * with e = 0 this is the Medusa draft on the same tree.
"""

import numpy as np

from .bf16 import round_bf16
from .heads import head_hidden, lm_project
from .topk import topk_stable


def hydra_draft(h, E, W, LM, k, plan, root, bf16=True, parent_tokens=None):
    """Draft tokens of one sequence on the tree `plan`.

    h [H], E [V, H], W [K, H, H] ([head, out, in]), LM [V, H]; root: the root
    token.  parent_tokens (optional, [T]): take the token of every parent node
    from here instead of from this draft (to check one depth on another
    implementation's tokens).  Returns (tokens [T], logits {p: row [V]} for
    every node p whose children were drawn).
    """
    h = np.asarray(h, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    T = plan.T
    tokens = np.full(T, -1, dtype=np.int64)
    tokens[0] = int(root)
    logits = {}
    src = tokens if parent_tokens is None else np.asarray(parent_tokens)
    for c in range(1, T):
        p = int(plan.parent[c])
        d = int(plan.depth[c])
        if p not in logits:
            y = h + E[int(src[p])]
            if bf16:
                y = round_bf16(y)
            u = head_hidden(y[None, :], np.asarray(W)[d - 1 : d], bf16)[0, 1]
            row = lm_project(u[None, :], LM)[0]
            logits[p] = (row, topk_stable(row, k[d - 1]))
        tokens[c] = int(logits[p][1][plan.tuples[c][-1]])
    return tokens, {p: v[0] for p, v in logits.items()}
