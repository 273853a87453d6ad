"""Medusa heads and the shared LM projection (oracle; test infrastructure only).

aicassindra.com "Medusa deep dive", section "The heads are residual blocks,
not linear layers": a head is one residual block applied to the last hidden
state h_t, then the language-model projection,
    head_i(h_t) = LMproj(h_t + SiLU(W_i . h_t)),
and all heads run in parallel off the same h_t.  The same page ("What this
deep dive assumes") and zackli.ai "Speculative Decoding Deep Dive II"
(section "Medusa", the training formula with Head_0) fix the indexing: the
base model's own head ("Head 0") is LMproj(h_t) and owns t+1, Medusa head i
owns t+i+1.  Head 0 is exactly the W_i = 0 case of the formula.

Readings taken where the pages are silent:
  * no bias in W_i or in LMproj, no final norm (none is shown);
  * SiLU(z) = z * sigmoid(z);
  * W_i is stored [out, in] (row-major), LMproj is stored [V, H];
  * bf16 mode stores u = h + SiLU(W_i h) rounded to bf16 (the next matmul
    reads bf16 operands); logits are kept unrounded (float64 here, float32
    on the device).
"""

import numpy as np

from .bf16 import round_bf16


def silu(z):
    """SiLU(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def lm_project(x, LM):
    """logits[r, v] = sum_j LM[v, j] * x[r, j]   (float64).

    The shared language-model projection of the deep-dive head formula; on the
    verify pass the same projection is the base model's original output head
    (inferensys.com "Medusa Heads", verification phase).
    """
    x = np.asarray(x, dtype=np.float64)
    LM = np.asarray(LM, dtype=np.float64)
    return x @ LM.T


def head_hidden(h, W, bf16):
    """u[b, 0] = h[b];  u[b, i] = h[b] + SiLU(W_{i-1} h[b]) for i = 1..K.

    h: [b, H], W: [K, H, H] ([head, out, in]) or None (K = 0).
    Returns u: [b, K+1, H] float64 (rounded to bf16 values when bf16).
    """
    h = np.asarray(h, dtype=np.float64)
    b, H = h.shape
    K = 0 if W is None else W.shape[0]
    u = np.empty((b, K + 1, H), dtype=np.float64)
    u[:, 0, :] = h
    for i in range(K):
        Wi = np.asarray(W[i], dtype=np.float64)          # [out, in]
        z = h @ Wi.T                                      # z[b, o] = sum_j W[o, j] h[b, j]
        u[:, i + 1, :] = h + silu(z)
    if bf16:
        u = round_bf16(u)
    return u


def heads(h, W, LM, bf16):
    """All K+1 head distributions' logits from one hidden state per sequence.

    Returns (u [b, K+1, H], logits [b, K+1, V]); row 0 is the base head.
    """
    u = head_hidden(h, W, bf16)
    b, K1, H = u.shape
    logits = lm_project(u.reshape(b * K1, H), LM).reshape(b, K1, -1)
    return u, logits
