"""Pins of exact rejection-sampling acceptance (oracle.accept_reject).

The defining property (aiunderstanding.org "Medusa Decoding Heads", "Deep
Dive": rejection sampling keeps the original model's output distribution):
each token emitted by a step is distributed as the model's tempered
distribution at its position.  Checked by counting over many seeds on a tiny
tree and vocabulary, against softmax(row / T) computed here; plus the
deterministic extremes (a certain candidate is always taken; candidates of
zero probability are never taken and never drawn as the next token).
"""

import numpy as np

from oracle import accept_reject

PARENT = np.array([-1, 0, 0, 1, 1, 2])
TOKENS = np.array([5, 1, 3, 0, 2, 4])     # node tokens (node 0 = root)
K, V = 2, 6
TEMP = float(np.float32(0.7))


def _p(row):
    x = np.asarray(row, dtype=np.float64) / TEMP
    e = np.exp(x - x.max())
    return e / e.sum()


def _emitted(logits, seed):
    L, path, acc, bonus, _ = accept_reject(logits, TOKENS, PARENT, K, TEMP, seed, 3, 1)
    out = [int(t) for t in acc[1 : L + 1]] + [int(bonus)]
    return out, [int(n) for n in path[: L + 1]]


def _close(counts, p, n):
    freq = counts / n
    sd = np.sqrt(p * (1 - p) / n)
    return np.all(np.abs(freq - p) <= 5 * sd + 2e-3)


def test_emitted_tokens_follow_the_model_distribution():
    rng = np.random.default_rng(2024)
    logits = rng.normal(0.0, 1.2, size=(len(TOKENS), V))
    logits[0] = [0.2, 1.0, -0.3, 0.8, -1.0, 0.1]   # both root candidates likely
    n = 60000
    first = np.zeros(V)
    second = {1: np.zeros(V), 2: np.zeros(V)}      # after taking node 1 / node 2
    taken = {1: 0, 2: 0}
    for seed in range(n):
        toks, path = _emitted(logits, seed)
        first[toks[0]] += 1
        if len(path) >= 2:
            c = path[1]
            taken[c] += 1
            second[c][toks[1]] += 1
    assert _close(first, _p(logits[0]), n)
    for c in (1, 2):
        assert taken[c] > 3000
        assert _close(second[c], _p(logits[c]), taken[c])


def test_certain_candidates_are_always_taken():
    logits = np.zeros((len(TOKENS), V))
    logits[0, 1] = 60.0          # root: node 1 (token 1) certain
    logits[1, 2] = 60.0          # node 1: its second child, node 4 (token 2), certain
    logits[4, 5] = 60.0          # leaf node 4: the next token is 5
    for seed in range(200):
        L, path, acc, bonus, _ = accept_reject(logits, TOKENS, PARENT, K, TEMP, seed, 0, 0)
        assert L == 2 and list(path) == [0, 1, 4] and list(acc) == [5, 1, 2] and bonus == 5


def test_impossible_candidates_are_never_taken_nor_drawn():
    logits = np.random.default_rng(7).normal(0.0, 1.0, size=(len(TOKENS), V))
    logits[0, 1] = logits[0, 3] = -1e4   # both root candidates have probability 0
    seen = set()
    for seed in range(500):
        L, path, _, bonus, _ = accept_reject(logits, TOKENS, PARENT, K, TEMP, seed, 0, 0)
        assert L == 0 and path[0] == 0 and path[1] == -1
        assert bonus not in (1, 3)
        seen.add(int(bonus))
    assert seen == {0, 2, 4, 5}
