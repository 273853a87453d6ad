"""MTP-style draft heads: one transformer layer per head (oracle; test infra only).

zackli.ai "Speculative Decoding Deep Dive II: Medusa, MTP", section "MTP":
multi-token prediction keeps the Medusa layout -- one shared trunk, n heads
on h_t, one shared unembedding f_u -- with
    P(x_{t+i} | x_{<=t}) = softmax(f_u(f_{h_i}(h_t))),  i = 1..n,
where each head f_{h_i} is a transformer layer rather than a single MLP; the
drafts then go through the same tree verification as Medusa heads.

The page fixes no layer shape.  Reading taken (the plainest one the rest
supports): f_{h_i} is one pre-norm transformer layer of the trunk's own kind
(the workloads name Llama shapes), applied at the current position t:
    a  = RMSNorm(h; g1_i)                      RMSNorm(x; g) = x / sqrt(mean(x^2) + eps) * g
    q, k, v = a Wq_i^T, a Wk_i^T, a Wv_i^T     (nq, nkv heads of dim d)
    o  = softmax(q k^T / sqrt(d)) v            over the head's own cache of the prefix
                                               [0, P) and the current position (k, v)
    x1 = h + o Wo_i^T
    a2 = RMSNorm(x1; g2_i)
    y  = x1 + (SiLU(a2 Wg_i^T) * (a2 Wu_i^T)) Wd_i^T     (SwiGLU MLP of width F)
    logits_i = LM y                            (f_u = the shared LM projection)
The head's cache holds K/V of the earlier positions (inputs here, as the
trunk's own cache is for tree attention: the layers that would write them need
trained weights).  Query head h reads kv head floor(h * nkv / nq).  bf16 mode
rounds to bf16 where the device stores a value (a, q, k, v, o, x1, a2, the
SwiGLU product, y), float64 elsewhere.  Head 0 is the base head, LM h.
"""

import numpy as np

from .bf16 import round_bf16
from .heads import silu


def rmsnorm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g along the last axis (float64)."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + float(eps))
    return x * r * np.asarray(g, dtype=np.float64)


def mtp_head(h, g1, Wq, Wk, Wv, Wo, g2, Wg, Wu, Wd, Kc, Vc, P, nq, nkv, eps, bf16):
    """One MTP head at the current position for a batch.

    h [b, H]; g1, g2 [H]; Wq [nq d, H]; Wk, Wv [nkv d, H]; Wo [H, nq d];
    Wg, Wu [F, H]; Wd [H, F]; Kc, Vc [b, nkv, >= P, d] (the head's cache,
    positions [0, P) used); P [b].  Returns y [b, H] and the current
    position's (k, v) [b, nkv, d] (what the head appends to its cache).
    """
    rnd = round_bf16 if bf16 else (lambda x: x)
    h = np.asarray(h, dtype=np.float64)
    b, H = h.shape
    d = np.asarray(Wq).shape[0] // nq
    a = rnd(rmsnorm(h, g1, eps))
    q = rnd(a @ np.asarray(Wq, dtype=np.float64).T).reshape(b, nq, d)
    k = rnd(a @ np.asarray(Wk, dtype=np.float64).T).reshape(b, nkv, d)
    v = rnd(a @ np.asarray(Wv, dtype=np.float64).T).reshape(b, nkv, d)
    o = np.empty((b, nq, d))
    scale = 1.0 / np.sqrt(d)
    for s in range(b):
        p = int(P[s])
        for hq in range(nq):
            g = (hq * nkv) // nq
            keys = np.concatenate([np.asarray(Kc[s, g, :p], dtype=np.float64), k[s, g][None]])
            vals = np.concatenate([np.asarray(Vc[s, g, :p], dtype=np.float64), v[s, g][None]])
            sc = keys @ q[s, hq] * scale
            e = np.exp(sc - sc.max())
            o[s, hq] = (e @ vals) / e.sum()
    o = rnd(o.reshape(b, nq * d))
    x1 = rnd(h + o @ np.asarray(Wo, dtype=np.float64).T)
    a2 = rnd(rmsnorm(x1, g2, eps))
    z = rnd(silu(a2 @ np.asarray(Wg, dtype=np.float64).T) * (a2 @ np.asarray(Wu, dtype=np.float64).T))
    y = rnd(x1 + z @ np.asarray(Wd, dtype=np.float64).T)
    return y, k, v


def mtp_draft(h, heads, LM, Kh, Vh, P, nq, nkv, eps, bf16):
    """All K MTP heads and the base head from one hidden state per sequence.

    heads: list of K dicts with g1, Wq, Wk, Wv, Wo, g2, Wg, Wu, Wd; Kh, Vh:
    [K, b, nkv, >= P, d].  Returns u [b, K+1, H] (slot 0 = h, slot i = head
    i's y), logits [b, K+1, V] = LM u, and the appended (k, v) per head.
    """
    h = np.asarray(h, dtype=np.float64)
    b, H = h.shape
    K = len(heads)
    u = np.empty((b, K + 1, H))
    u[:, 0] = h
    kv = []
    for i, w in enumerate(heads):
        y, k, v = mtp_head(h, w["g1"], w["Wq"], w["Wk"], w["Wv"], w["Wo"], w["g2"], w["Wg"],
                           w["Wu"], w["Wd"], Kh[i], Vh[i], P, nq, nkv, eps, bf16)
        u[:, i + 1] = y
        kv.append((k, v))
    logits = (u.reshape(b * (K + 1), H) @ np.asarray(LM, dtype=np.float64).T).reshape(b, K + 1, -1)
    return u, logits, kv
