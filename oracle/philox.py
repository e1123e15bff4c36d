"""Philox4x32-10 and the verify step's per-position uniforms (oracle side).

Philox is defined in Salmon, Moraes, Dror & Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3" (SC'11), section on Philox: a 4x32-bit counter and a 2x32-bit
key; each round multiplies counter words 0 and 2 by two fixed odd constants,
splits the 64-bit products into high and low halves, and recombines them with
the other two words and the round key; the key advances by the two Weyl
constants (golden ratio and sqrt(3)-1, times 2^32) between rounds. Ten rounds.

How the verify step keys it (the pages only say uniforms must not change the
target distribution; the keying is this build's reading):

* key     = (seed mod 2^32, seed >> 32)
* counter = (pos, seq_id mod 2^32, seq_id >> 32, stream)   stream 0 = verify
* u_acc   = (word0 >> 8) * 2^-24,  u_smp = (word1 >> 8) * 2^-24

``pos`` is the absolute position of the token being decided, so every
(sequence, position) is decided with fresh uniforms exactly once over a rollout.
"""

from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
# Round multipliers and key increments of Philox4x32 (SC'11, Philox parameters).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10


def philox4x32_10(counter, key):
    """Scalar reference: counter is 4 uint32 ints, key is 2 uint32 ints; returns 4 uint32 ints."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in counter)
    k0, k1 = (int(x) & MASK32 for x in key)
    for r in range(ROUNDS):
        if r > 0:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        prod0 = PHILOX_M0 * c0
        prod1 = PHILOX_M1 * c2
        hi0, lo0 = prod0 >> 32, prod0 & MASK32
        hi1, lo1 = prod1 >> 32, prod1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return c0, c1, c2, c3


def philox4x32_10_np(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10 over uint32 arrays (broadcasting); returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & MASK32
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for r in range(ROUNDS):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & np.uint64(MASK32)
            k1 = (k1 + np.uint64(PHILOX_W1)) & np.uint64(MASK32)
        prod0 = m0 * c0          # < 2^64, exact in uint64
        prod1 = m1 * c2
        hi0, lo0 = prod0 >> np.uint64(32), prod0 & np.uint64(MASK32)
        hi1, lo1 = prod1 >> np.uint64(32), prod1 & np.uint64(MASK32)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def _split64(x: int):
    x = int(x) & 0xFFFFFFFFFFFFFFFF
    return x & MASK32, x >> 32


def word_to_unit(w) -> float:
    """Top 24 bits of a uint32 word as a multiple of 2^-24 in [0, 1 - 2^-24]."""
    return (int(w) >> 8) * (2.0 ** -24)


def verify_uniforms(seed: int, seq_id: int, pos: int, stream: int = 0):
    """(u_acc, u_smp) for deciding the token at absolute position ``pos`` of sequence ``seq_id``."""
    k0, k1 = _split64(seed)
    s0, s1 = _split64(seq_id)
    w = philox4x32_10((int(pos) & MASK32, s0, s1, stream), (k0, k1))
    return word_to_unit(w[0]), word_to_unit(w[1])


def verify_uniforms_np(seed: int, seq_ids, positions, stream: int = 0):
    """Vectorised (u_acc, u_smp) arrays for broadcast arrays of sequence ids and positions."""
    k0, k1 = _split64(seed)
    sid = np.asarray(seq_ids, dtype=np.int64).astype(np.uint64)
    pos = np.asarray(positions, dtype=np.int64).astype(np.uint64) & np.uint64(MASK32)
    w0, w1, _, _ = philox4x32_10_np(pos, sid & np.uint64(MASK32), sid >> np.uint64(32),
                                    np.uint64(stream), k0, k1)
    scale = 2.0 ** -24
    return (w0 >> np.uint32(8)).astype(np.float64) * scale, (w1 >> np.uint32(8)).astype(np.float64) * scale
