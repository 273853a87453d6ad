"""bfloat16 rounding for the oracle (test infrastructure only).

The bf16 path stores two intermediates in bf16: the head hidden state u and
the attention output O.  The oracle mirrors those two stored roundings and is
float64 everywhere else.  bfloat16 keeps the top 16 bits of an IEEE binary32;
rounding is to nearest, ties to even.  Pinned against torch's own float->bf16
conversion in ``tests/test_oracle_numerics.py``.
"""

import numpy as np


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value (ties to even).

    The value is first rounded to binary32 (as a float32 store would), then
    the low 16 bits of the binary32 pattern are rounded away.  Returns float64.
    Inputs must be finite.
    """
    a = np.asarray(x, dtype=np.float64)
    f = a.astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = (bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = (rounded << np.uint64(16)).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)
