"""Philox-4xW-10 counter-based generator of the oracle (test infrastructure only).

Published method: J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11, section 4 (the Philox family).  A Philox
bijection maps a 4-word counter under a 2-word key through R rounds.  One round
multiplies counter words 0 and 2 by two fixed odd constants, keeps both halves
of each double-width product, and permutes:

    (hi0, lo0) = M0 * c0          (hi1, lo1) = M1 * c2
    c' = (hi1 ^ c1 ^ k0,  lo1,  hi0 ^ c3 ^ k1,  lo0)

Between rounds the key advances by two Weyl constants, (k0, k1) += (W0, W1),
taken from the golden ratio and sqrt(3):  W0 = floor(2^W * (phi - 1)),
W1 = floor(2^W * (sqrt(3) - 1)).  Philox-4xW-10 runs 10 rounds (the key is
advanced 9 times).

Two implementations live here:
  * ``philox_ref`` -- pure-Python integers, any word width (32 or 64).  The
    64-bit instance is checked against numpy's ``Philox`` bit generator (a
    library implementation of Philox-4x64-10), which fixes the round structure
    (operand order, permutation, key schedule, round count).
  * ``philox4x32_10`` -- the vectorised 32-bit instance used by the region
    oracle; checked against ``philox_ref`` at W = 32.
"""
from __future__ import annotations

import numpy as np

# Multipliers and Weyl increments from the paper, per word width.
PHILOX_CONSTANTS = {
    32: dict(M0=0xD2511F53, M1=0xCD9E8D57, W0=0x9E3779B9, W1=0xBB67AE85),
    64: dict(M0=0xD2E7470EE14C6C93, M1=0xCA5A826395121157,
             W0=0x9E3779B97F4A7C15, W1=0xBB67AE8584CAA73B),
}


def philox_ref(counter, key, width=32, rounds=10):
    """Philox-4x``width``-``rounds`` on Python ints: counter = 4 words, key = 2 words."""
    c = PHILOX_CONSTANTS[width]
    mask = (1 << width) - 1
    c0, c1, c2, c3 = (int(x) & mask for x in counter)
    k0, k1 = (int(x) & mask for x in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + c["W0"]) & mask
            k1 = (k1 + c["W1"]) & mask
        p0 = c["M0"] * c0
        p1 = c["M1"] * c2
        hi0, lo0 = p0 >> width, p0 & mask
        hi1, lo1 = p1 >> width, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return (c0, c1, c2, c3)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox-4x32-10.  Arguments are broadcastable integer arrays
    holding 32-bit words; returns four uint32 arrays."""
    M0 = np.uint64(PHILOX_CONSTANTS[32]["M0"])
    M1 = np.uint64(PHILOX_CONSTANTS[32]["M1"])
    W0 = np.uint64(PHILOX_CONSTANTS[32]["W0"])
    W1 = np.uint64(PHILOX_CONSTANTS[32]["W1"])
    mask = np.uint64(0xFFFFFFFF)
    sh = np.uint64(32)
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & mask for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & mask
    k1 = np.asarray(k1, dtype=np.uint64) & mask
    for r in range(10):
        if r:
            k0 = (k0 + W0) & mask
            k1 = (k1 + W1) & mask
        p0 = M0 * c0          # < 2^64: exact in uint64
        p1 = M1 * c2
        c0, c1, c2, c3 = (p1 >> sh) ^ c1 ^ k0, p1 & mask, (p0 >> sh) ^ c3 ^ k1, p0 & mask
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))
