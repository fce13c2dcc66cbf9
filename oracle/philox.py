"""Philox4x32-10, written from its published description (oracle side; test infrastructure).

Source: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random Numbers:
As Easy as 1, 2, 3", SC'11, the Philox-4x32 bijection with 10 rounds.

State: a counter of four 32-bit words (c0, c1, c2, c3) and a key of two 32-bit words
(k0, k1).  One round takes the two 64-bit products M0*c0 and M1*c2, each split into a
high and a low 32-bit word, and forms the new counter

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0)).

Between rounds the key is bumped by the Weyl increments (W0, W1), modulo 2^32.  The
counter after the tenth round is the output block of four 32-bit words.

Two independent implementations live here: ``block_scalar`` uses Python integers one
block at a time; ``blocks_np`` is vectorized over numpy arrays with 64-bit products.
They are checked against each other and against the closed forms of the constants.
"""
from __future__ import annotations

import numpy as np

# Multipliers given in the paper for Philox-4x32.
M0 = 0xD2511F53
M1 = 0xCD9E8D57
# Weyl key increments: the fractional parts of the golden ratio and of sqrt(3), scaled
# by 2^32 and truncated.  Tests re-derive both from those closed forms.
W0 = 0x9E3779B9
W1 = 0xBB67AE85
ROUNDS = 10
_MASK32 = 0xFFFFFFFF


def block_scalar(counter, key):
    """One Philox4x32-10 block; ``counter`` is 4 ints, ``key`` 2 ints (all < 2**32)."""
    c0, c1, c2, c3 = (int(v) & _MASK32 for v in counter)
    k0, k1 = (int(v) & _MASK32 for v in key)
    for r in range(ROUNDS):
        p0 = M0 * c0
        p1 = M1 * c2
        hi0, lo0 = p0 >> 32, p0 & _MASK32
        hi1, lo1 = p1 >> 32, p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        if r != ROUNDS - 1:
            k0 = (k0 + W0) & _MASK32
            k1 = (k1 + W1) & _MASK32
    return (c0, c1, c2, c3)


def blocks_np(c0, c1, c2, c3, k0, k1):
    """Vectorized Philox4x32-10 over uint32 arrays (counters) and scalar key words.

    Returns a uint32 array of shape (n, 4): the output block of each counter.
    """
    c0 = np.asarray(c0, dtype=np.uint32)
    n = c0.shape[0]
    c1 = np.broadcast_to(np.asarray(c1, dtype=np.uint32), (n,)).copy()
    c2 = np.broadcast_to(np.asarray(c2, dtype=np.uint32), (n,)).copy()
    c3 = np.broadcast_to(np.asarray(c3, dtype=np.uint32), (n,)).copy()
    c0 = c0.copy()
    k0 = int(k0) & _MASK32
    k1 = int(k1) & _MASK32
    m0 = np.uint64(M0)
    m1 = np.uint64(M1)
    sh = np.uint64(32)
    for r in range(ROUNDS):
        p0 = c0.astype(np.uint64) * m0
        p1 = c2.astype(np.uint64) * m1
        hi0 = (p0 >> sh).astype(np.uint32)
        lo0 = p0.astype(np.uint32)
        hi1 = (p1 >> sh).astype(np.uint32)
        lo1 = p1.astype(np.uint32)
        n0 = hi1 ^ c1 ^ np.uint32(k0)
        n2 = hi0 ^ c3 ^ np.uint32(k1)
        c0, c1, c2, c3 = n0, lo1, n2, lo0
        if r != ROUNDS - 1:
            k0 = (k0 + W0) & _MASK32
            k1 = (k1 + W1) & _MASK32
    return np.stack([c0, c1, c2, c3], axis=1)
