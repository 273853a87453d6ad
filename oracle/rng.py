"""Counter-based sampler draws (oracle; test infrastructure only).

The pages ask for a seeded sampler for the root and the next ("bonus") token
in typical-acceptance mode but fix no generator.  Reading taken: one integer
counter-based generator, SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; the public-domain reference
``splitmix64.c`` by S. Vigna), evaluated statelessly:

    x = splitmix64(seed ^ (step << 32) ^ (seq << 8) ^ draw)     (mod 2**64)
    u = (x >> 40) * 2**-24                                        in [0, 1)

where splitmix64(z) is the first output of a SplitMix64 stream whose state
is z.  draw 0 = root token, draw 1 = bonus token.  The device side implements
the same published definition independently; u is therefore bit-identical.

Sampling from q = softmax(x / T): e_i = exp((x_i - max x) / T), S = sum e,
the sample is the smallest i whose running sum (ascending vocabulary order)
exceeds u * S.
"""

import numpy as np

_MASK = (1 << 64) - 1


def splitmix64(z):
    """First output of a SplitMix64 stream with state z (Python ints, exact)."""
    z = (z + 0x9E3779B97F4A7C15) & _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def counter_uniform(seed, step, seq, draw):
    """u in [0, 1) with 24 random bits, from the counter (seed, step, seq, draw)."""
    ctr = (seed ^ ((step << 32) & _MASK) ^ (seq << 8) ^ draw) & _MASK
    x = splitmix64(ctr)
    return (x >> 40) * (2.0 ** -24)


def sample_tempered(row, temperature, u):
    """Inverse-CDF sample from softmax(row / temperature), float64.

    ``temperature`` is used as given (the device receives it as float32, so the
    caller passes the float32 value).  Returns (index, cdf) where cdf is the
    unnormalised running sum, for margin checks.
    """
    x = np.asarray(row, dtype=np.float64)
    m = x.max()
    e = np.exp((x - m) / float(temperature))
    c = np.cumsum(e)
    target = u * c[-1]
    i = int(np.searchsorted(c, target, side="right"))
    return min(i, x.size - 1), c
