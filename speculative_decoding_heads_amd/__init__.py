"""Medusa draft-and-verify step on AMD Instinct MI355X (gfx950).

The step runs in hand-written HIP kernels behind the C ABI of
``libmedusa.so`` (declared in ``include/medusa.h``).  ``speculative_decoding_heads_amd.medusa``
is the thin Python binding (argument marshalling only); ``configs`` and
``synth`` describe and draw the synthetic workloads.  Importing this package
does not load the library; the first binding call does, and raises if the
library is missing.
"""

__all__ = ["configs", "synth", "medusa"]
