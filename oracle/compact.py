"""Rollback / compaction of the speculative KV entries (oracle; test infra).

inferensys.com "Medusa Heads": after verification the process rolls back to
the last accepted position; the speculative KV cache manages the key/value
entries of the candidate tree.

Reading: the tree nodes' K/V occupy cache slots P .. P+T-1 in node order.
After acceptance the entries of the accepted path (node path[d] at depth d)
move to slots P + d, d = 0..L, for every kv head, K and V alike; the new
sequence length is P + L + 1 (root + L accepted candidates).  Slots at or past
the new length are stale.  The move is defined on a snapshot of the cache
(read every source, then write).
"""

import numpy as np


def kv_compact(Kc, Vc, P, path, L):
    """One sequence: Kc, Vc [nkv, Pmax, d].  Returns (Kc', Vc', new_len)."""
    K0 = np.array(Kc, copy=True)
    V0 = np.array(Vc, copy=True)
    Kn = np.array(Kc, copy=True)
    Vn = np.array(Vc, copy=True)
    for d in range(L + 1):
        src = P + int(path[d])
        Kn[:, P + d] = K0[:, src]
        Vn[:, P + d] = V0[:, src]
    return Kn, Vn, P + L + 1
