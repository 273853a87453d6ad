"""Greedy and typical acceptance, path choice and next token (oracle).

Test infrastructure only.

Pages:
  * aiunderstanding.org "Medusa Decoding Heads", "Deep Dive": the model
    verifies the whole tree in one pass and accepts the longest prefix that
    matches what it would have produced anyway (greedy).
  * inferensys.com "Medusa Heads": verification stops at the first rejected
    token; rollback to the last accepted position; the next token comes from
    the base model.
  * aicassindra.com "Medusa deep dive", "Typical acceptance, not exact
    rejection sampling": accept a proposed token when the model's probability
    for it exceeds min(eps, delta * exp(-H)), H the entropy of the model's
    distribution at that step.

Readings:
  * greedy: argmax ties go to the lowest vocabulary index;
  * typical: the model distribution is softmax(logits / T) (the tempered
    distribution), H uses the natural log, the comparison is strict '>';
  * a node is fully accepted when it and all its ancestors below the root are
    accepted; L = the largest depth of a fully accepted node (0..K); the chosen
    node is the lowest node index among fully accepted nodes at depth L;
  * next ("bonus") token at the chosen node: argmax (greedy) or a seeded
    sample from softmax(logits / T) (typical; draw 1 of the counter sampler);
  * path = node indices root .. chosen node, padded with -1 to K+1 entries;
    accepted tokens likewise.

Exact rejection sampling (accept_reject).  aiunderstanding.org "Medusa
Decoding Heads" ("Deep Dive"): with the backbone frozen, rejection sampling
against the original model can keep its output distribution (lossless);
aicassindra.com "Medusa deep dive", "Typical acceptance, not exact rejection
sampling": the heads give no clean proposal distribution to reject against.
Reading: the candidates of a node are taken as point-mass proposals, tried in
node order.  At node n with tempered distribution p_n = softmax(row_n / T),
child j (token t_j) is accepted when u_j * (1 - r_j) < p_n(t_j), r_j the mass
of the children already rejected (p_n(t_1) + ... + p_n(t_{j-1})); the walk
moves to the first accepted child.  When every child of n is rejected, the
next token is drawn from p_n with those children's tokens removed (inverse
CDF on the remaining mass, draw 1); when n has no children, from p_n itself.
Each emitted token is then distributed exactly as p at its position: child j
is emitted with probability p(t_j) and the residual covers the rest.  Draws:
u_j of the child at index j among the children of a depth-d node is draw
16 d + j of the counter sampler keyed by splitmix64(seed) (separate from the
root and bonus draws keyed by seed).
"""

import numpy as np

from .rng import counter_uniform, sample_tempered, splitmix64


def _path_to(best, parent, K):
    chain = []
    j = best
    while j >= 0:
        chain.append(j)
        j = int(parent[j])
    chain.reverse()
    path = np.full(K + 1, -1, dtype=np.int64)
    path[: len(chain)] = chain
    return path


def accept_greedy_walk(base_logits, tokens, parent, K):
    """Token-by-token replay: follow the child whose token is the argmax.

    base_logits: [T, V] for one sequence; tokens: [T]; parent: [T].
    Returns (L, path[K+1], acc_tokens[K+1], bonus).
    """
    T = len(tokens)
    children = [[] for _ in range(T)]
    for c in range(1, T):
        children[int(parent[c])].append(c)
    cur, L = 0, 0
    while True:
        want = int(np.argmax(np.asarray(base_logits[cur], dtype=np.float64)))
        nxt = [c for c in children[cur] if int(tokens[c]) == want]
        if not nxt:
            break
        cur = nxt[0]
        L += 1
    path = _path_to(cur, parent, K)
    acc = np.where(path >= 0, np.asarray(tokens)[np.maximum(path, 0)], -1)
    return L, path, acc, want


def _select(full, depth, parent, tokens, K):
    T = len(full)
    L = max(int(depth[i]) for i in range(T) if full[i])
    best = min(i for i in range(T) if full[i] and int(depth[i]) == L)
    path = _path_to(best, parent, K)
    acc = np.where(path >= 0, np.asarray(tokens)[np.maximum(path, 0)], -1)
    return L, best, path, acc


def _full_flags(local, parent):
    T = len(local)
    full = np.zeros(T, dtype=bool)
    full[0] = True
    for c in range(1, T):                    # parent index < child index
        full[c] = bool(local[c]) and full[int(parent[c])]
    return full


def accept_greedy_parallel(base_logits, tokens, parent, depth, K):
    """Parallel form: local match flags, full-path flags, deepest full node."""
    T = len(tokens)
    amax = [int(np.argmax(np.asarray(base_logits[i], dtype=np.float64))) for i in range(T)]
    local = np.zeros(T, dtype=bool)
    for c in range(1, T):
        local[c] = int(tokens[c]) == amax[int(parent[c])]
    full = _full_flags(local, parent)
    L, best, path, acc = _select(full, depth, parent, tokens, K)
    return L, path, acc, amax[best]


def typical_local(row, token, temperature, eps, delta):
    """Typical test for one candidate token against one parent distribution.

    Returns (accepted, q_token, threshold, entropy), all float64.
    """
    x = np.asarray(row, dtype=np.float64) / float(temperature)
    x = x - x.max()
    e = np.exp(x)
    q = e / e.sum()
    nz = q > 0
    H = float(-(q[nz] * np.log(q[nz])).sum())
    thr = min(float(eps), float(delta) * np.exp(-H))
    qt = float(q[int(token)])
    return qt > thr, qt, thr, H


def accept_typical(base_logits, tokens, parent, depth, K, temperature, eps, delta,
                   seed, step, seq):
    """Typical acceptance for one sequence.

    Returns (L, path, acc_tokens, bonus, margins) where margins[c] is
    |q - thr| / thr of each candidate's decision (for near-tie accounting).
    """
    T = len(tokens)
    local = np.zeros(T, dtype=bool)
    margins = np.full(T, np.inf)
    for c in range(1, T):
        ok, qt, thr, _ = typical_local(base_logits[int(parent[c])], tokens[c],
                                       temperature, eps, delta)
        local[c] = ok
        margins[c] = abs(qt - thr) / thr
    full = _full_flags(local, parent)
    L, best, path, acc = _select(full, depth, parent, tokens, K)
    u = counter_uniform(seed, step, seq, 1)
    bonus, _ = sample_tempered(base_logits[best], temperature, u)
    return L, path, acc, bonus, margins


def accept_reject(base_logits, tokens, parent, K, temperature, seed, step, seq):
    """Exact rejection sampling over the tree for one sequence.

    Returns (L, path, acc_tokens, bonus, margins): margins lists, for every
    decision taken, |u (1 - r) - p| / p (near-tie accounting; inf when p = 0).
    """
    T = len(tokens)
    children = [[] for _ in range(T)]
    for c in range(1, T):
        children[int(parent[c])].append(c)

    def probs(n):
        x = np.asarray(base_logits[n], dtype=np.float64) / float(temperature)
        e = np.exp(x - x.max())
        return e / e.sum()

    seed_w = splitmix64(seed)
    n, d, margins = 0, 0, []
    rejected_all = False
    while children[n]:
        p = probs(n)
        r, nxt = 0.0, None
        for j, c in enumerate(children[n]):
            pc = float(p[int(tokens[c])])
            u = counter_uniform(seed_w, step, seq, 16 * d + j)
            lhs = u * (1.0 - r)
            margins.append(abs(lhs - pc) / pc if pc > 0 else np.inf)
            if lhs < pc:
                nxt = c
                break
            r += pc
        if nxt is None:
            rejected_all = True
            break
        n, d = nxt, d + 1
    L = d
    path = _path_to(n, parent, K)
    acc = np.array([int(tokens[i]) if i >= 0 else -1 for i in path], dtype=np.int64)
    x = np.asarray(base_logits[n], dtype=np.float64) / float(temperature)
    e = np.exp(x - x.max())
    if rejected_all:
        for c in children[n]:
            e[int(tokens[c])] = 0.0
    cdf = np.cumsum(e)
    u = counter_uniform(seed, step, seq, 1)
    bonus = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
    return L, path, acc, min(bonus, e.size - 1), margins
