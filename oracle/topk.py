"""Per-head top-k shortlist and greedy root (oracle; test infrastructure only).

aicassindra.com "Medusa deep dive", section "From top-k heads to a sparse
candidate tree": keep the top k_i tokens of head i; skandtandon "day 89",
section "Tree-based attention": each head predicts its top-k tokens.

Reading for ties (the pages are silent): order by logit descending, equal
logits by lower vocabulary index first; -0.0 and +0.0 are equal.  That is a
stable sort of the negated row, which this module uses directly.
"""

import numpy as np


def topk_stable(row, k):
    """Indices of the k largest entries, descending, ties to the lower index."""
    row = np.asarray(row, dtype=np.float64)
    order = np.argsort(-row, kind="stable")
    return order[:k].astype(np.int64)


def argmax_lowest(row):
    """Index of the largest entry; the lowest such index on ties."""
    row = np.asarray(row, dtype=np.float64)
    return int(np.argmax(row))
