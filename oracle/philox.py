"""Philox4x32-10 counter-based random numbers.

Test infrastructure only (see ``oracle/__init__``).

Definition followed: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), the Philox-4x32
bijection with 10 rounds.  A round maps the counter (c0, c1, c2, c3) under
the key (k0, k1) to

    (hi(M1 c2) ^ c1 ^ k0,  lo(M1 c2),  hi(M0 c0) ^ c3 ^ k1,  lo(M0 c0))

with the 32 x 32 -> 64-bit products split into high and low words,
M0 = 0xD2511F53 and M1 = 0xCD9E8D57; between rounds the key is bumped by the
Weyl constants (0x9E3779B9, 0xBB67AE85) modulo 2^32.  Written here from
that description with NumPy uint64 arithmetic, vectorised over counters.
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK = 0xFFFFFFFF
ROUNDS = 10


def philox4x32(c0, c1, c2, c3, k0: int, k1: int, rounds: int = ROUNDS):
    """Philox4x32 of counter words (arrays or ints, broadcast) under the key
    (k0, k1).  Returns four uint32 arrays."""
    c = [np.asarray(v, dtype=np.uint64) & MASK for v in (c0, c1, c2, c3)]
    c = np.broadcast_arrays(*c)
    c0, c1, c2, c3 = (v.copy() for v in c)
    k0, k1 = int(k0) & MASK, int(k1) & MASK
    for r in range(rounds):
        p0 = c0 * np.uint64(M0)                      # < 2^64: exact in uint64
        p1 = c2 * np.uint64(M1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK)
        c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
        k0, k1 = (k0 + W0) & MASK, (k1 + W1) & MASK
    return tuple(v.astype(np.uint32) for v in (c0, c1, c2, c3))
