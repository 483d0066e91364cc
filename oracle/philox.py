"""Philox-4xW counter-based generator (TEST INFRASTRUCTURE ONLY: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module; it shares no code with the GPU path).

Written from the published definition: J. K. Salmon, M. A. Moraes,
R. O. Dror and D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC 2011 (the Philox S-box and key schedule).  One round maps a counter of
four W-bit words (c0, c1, c2, c3) under a key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

where hi/lo are the upper and lower W bits of the 2W-bit product; between
rounds the key is advanced by the Weyl constants (k0 += W0, k1 += W1,
mod 2^W).  Philox4x32-10 (ten rounds, 32-bit words) drives the dropout
mask; the 64-bit instance is here only so that tests can hold the same
round code against numpy's Philox4x64-10 bit generator.

The function works on Python ints (any W) or on numpy uint64 arrays
(W = 32 only: the 64-bit product of two 32-bit words is exact).
"""
from __future__ import annotations

import numpy as np

# multipliers (the paper's table for N = 4) and Weyl key increments (the
# W-bit fractional parts of the golden ratio and of sqrt(3))
PARAMS = {
    32: (0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85),
    64: (0xD2E7470EE14C6C93, 0xCA5A826395121157, 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B),
}


def philox4(counter, key, width=32, rounds=10):
    """Philox-4x``width``-``rounds`` of one counter (or arrays of counters,
    broadcast together).  Returns the four output words."""
    M0, M1, W0, W1 = PARAMS[width]
    if width == 32:
        as_word = lambda x: np.asarray(x, dtype=np.uint64) & np.uint64(0xFFFFFFFF)
        mask, sh = np.uint64(0xFFFFFFFF), np.uint64(32)
        M0, M1, W0, W1 = (np.uint64(x) for x in (M0, M1, W0, W1))
    else:
        as_word = int
        mask, sh = (1 << width) - 1, width
    c0, c1, c2, c3 = (as_word(x) for x in counter)
    k0, k1 = (as_word(x) for x in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + W0) & mask
            k1 = (k1 + W1) & mask
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> sh) ^ c1 ^ k0, p1 & mask, (p0 >> sh) ^ c3 ^ k1, p0 & mask)
    return c0, c1, c2, c3
