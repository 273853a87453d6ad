"""Tree-masked attention of the verification pass (oracle; test infra only).

Pages:
  * inferensys.com "Medusa Heads", tree attention: every candidate branch
    shares the key/value cache of the common prefix, and all candidate nodes
    are scored in one pass.
  * aicassindra.com "Medusa deep dive", "From top-k heads to a sparse candidate
    tree": a node attends only to its own ancestors.
  * zackli.ai "Speculative Decoding Deep Dive II", "Medusa": Anc(i).

Readings (the pages give no attention formula of their own; this is plain
scaled dot-product attention): scale 1/sqrt(d); grouped query heads map q head
h to kv head floor(h * n_kv / n_q); no positional rotation (position ids are
produced but no encoding is named); node i sees prefix slots [0, P), itself
and its ancestors.  The tree nodes' K/V sit in cache slots P .. P+T-1.
bf16 mode stores O rounded to bf16.

Two independent routines:
  tree_attention  - one masked softmax over prefix + tree keys per node;
  path_attention  - for each node, the root-to-node path taken as its own
                    sequence after the prefix, plain causal attention, last row.
Their agreement is the central pin of this stage.
"""

import numpy as np

from .bf16 import round_bf16


def _kv_head(h, nq, nkv):
    return (h * nkv) // nq


def _softmax_attend(q, Ks, Vs, scale):
    """o = softmax(scale * Ks q) @ Vs, float64, max-subtracted."""
    s = (Ks @ q) * scale
    s = s - s.max()
    p = np.exp(s)
    return (p @ Vs) / p.sum()


def tree_attention(Q, Kc, Vc, P, anc, scale=None, bf16=False):
    """Masked-tree attention for a batch.

    Q: [b, T, nq, d]; Kc, Vc: [b, nkv, Pmax, d]; P: [b] prefix lengths;
    anc: [T, T] bool.  Returns O: [b, T, nq*d].
    """
    Q = np.asarray(Q, dtype=np.float64)
    b, T, nq, d = Q.shape
    nkv = Kc.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.empty((b, T, nq, d), dtype=np.float64)
    for s in range(b):
        p = int(P[s])
        for g in range(nkv):
            K = np.asarray(Kc[s, g, : p + T], dtype=np.float64)
            V = np.asarray(Vc[s, g, : p + T], dtype=np.float64)
            heads = [h for h in range(nq) if _kv_head(h, nq, nkv) == g]
            for t in range(T):
                vis = np.concatenate([np.ones(p, dtype=bool), anc[t]])
                for h in heads:
                    O[s, t, h] = _softmax_attend(Q[s, t, h], K[vis], V[vis], scale)
    O = O.reshape(b, T, nq * d)
    return round_bf16(O) if bf16 else O


def causal_attention_last(q, K, V, scale):
    """Plain causal attention of the last query position over a sequence.

    The last position of a causal sequence sees every earlier position and
    itself, so its output is the softmax over all keys of the sequence.
    """
    return _softmax_attend(q, K, V, scale)


def path_attention(Q, Kc, Vc, P, parent, scale=None, bf16=False):
    """Brute force: each node's path (root .. node) as its own sequence.

    For node t the sequence is the prefix K/V followed by the K/V of the
    nodes on the path root -> t (in path order); t is the last position.
    """
    Q = np.asarray(Q, dtype=np.float64)
    b, T, nq, d = Q.shape
    nkv = Kc.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    O = np.empty((b, T, nq, d), dtype=np.float64)
    for s in range(b):
        p = int(P[s])
        for t in range(T):
            chain = []
            j = t
            while j >= 0:
                chain.append(j)
                j = int(parent[j])
            chain.reverse()
            slots = list(range(p)) + [p + j for j in chain]
            for h in range(nq):
                g = _kv_head(h, nq, nkv)
                K = np.asarray(Kc[s, g, slots], dtype=np.float64)
                V = np.asarray(Vc[s, g, slots], dtype=np.float64)
                O[s, t, h] = causal_attention_last(Q[s, t, h], K, V, scale)
    O = O.reshape(b, T, nq * d)
    return round_bf16(O) if bf16 else O


def attention_row(q, Kc_sg, Vc_sg, P, anc_row, scale):
    """One output row (one node, one q head) for sampled checks at full size."""
    T = anc_row.shape[0]
    vis = np.concatenate([np.ones(P, dtype=bool), anc_row])
    K = np.asarray(Kc_sg[: P + T], dtype=np.float64)[vis]
    V = np.asarray(Vc_sg[: P + T], dtype=np.float64)[vis]
    return _softmax_attend(np.asarray(q, dtype=np.float64), K, V, scale)


def tree_attention_head(q, Kc_sg, Vc_sg, P, anc, scale):
    """Every node of one q head at once, as masked attention over a score matrix.

    q: [T, d] (the head's query of each node); Kc_sg, Vc_sg: [>= P+T, d] (the
    head's kv-head cache); anc: [T, T] bool.  S = scale * q K^T over all P+T
    keys, keys a node may not see set to -inf (prefix always visible, tree slot
    P+j visible iff anc[t, j]), row softmax, times V.  Returns [T, d] float64.
    The same quantity as tree_attention, written as one masked matrix product
    rather than a gather of the visible rows.
    """
    q = np.asarray(q, dtype=np.float64)
    T = q.shape[0]
    K = np.asarray(Kc_sg[: P + T], dtype=np.float64)
    V = np.asarray(Vc_sg[: P + T], dtype=np.float64)
    vis = np.concatenate([np.ones((T, P), dtype=bool), np.asarray(anc, dtype=bool)], axis=1)
    S = np.where(vis, (q @ K.T) * scale, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    E = np.exp(S)
    return (E @ V) / E.sum(axis=1, keepdims=True)
