"""Philox4x32-10 counter-based generator (oracle side).

Definition: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3", SC'11 -- the Philox-4x32 bijection with multipliers 0xD2511F53 and
0xCD9E8D57, Weyl key increments 0x9E3779B9 and 0xBB67AE85, 10 rounds.  One
round maps (c0, c1, c2, c3) with key (k0, k1) to
    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0));
the key is bumped by the Weyl constants between rounds.

Counter convention used by the drafter (the pages do not fix one; both the
sampler and the verifier draw their uniforms here):
    key     = (seed & 0xffffffff, seed >> 32)
    counter = (position, slot, step & 0xffffffff, purpose)
    u       = (out0 >> 8) * 2**-24          (exact in fp32 and fp64, in [0, 1))
purpose 0 = draft sampling, 1 = accept test, 2 = residual / bonus sample,
3 = synthetic target noise (benchmark only), 4 = draft-tree verifier walk.

Pinned by the published known-answer vectors (tests/golden/philox4x32_10_kat.txt).
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK = 0xFFFFFFFF

PURPOSE_DRAFT = 0
PURPOSE_ACCEPT = 1
PURPOSE_RESAMPLE = 2
PURPOSE_TREE_WALK = 4


def philox4x32(c0, c1, c2, c3, k0, k1, rounds: int = 10):
    """Vectorised Philox4x32-R over numpy arrays of counters; returns 4 uint64 arrays (< 2**32)."""
    c0 = np.asarray(c0, dtype=np.uint64) & MASK
    c1 = np.asarray(c1, dtype=np.uint64) & MASK
    c2 = np.asarray(c2, dtype=np.uint64) & MASK
    c3 = np.asarray(c3, dtype=np.uint64) & MASK
    k0 = np.uint64(int(k0) & MASK)
    k1 = np.uint64(int(k1) & MASK)
    m0, m1, mask = np.uint64(M0), np.uint64(M1), np.uint64(MASK)
    s32 = np.uint64(32)
    for r in range(rounds):
        p0 = m0 * c0
        p1 = m1 * c2
        c0, c1, c2, c3 = ((p1 >> s32) ^ c1 ^ k0), (p1 & mask), ((p0 >> s32) ^ c3 ^ k1), (p0 & mask)
        k0 = np.uint64((int(k0) + W0) & MASK)
        k1 = np.uint64((int(k1) + W1) & MASK)
    return c0, c1, c2, c3


def uniform(seed: int, slot, step: int, position, purpose: int):
    """u in [0,1) with 24 random bits for (seed; position, slot, step, purpose)."""
    seed = int(seed)
    position = np.asarray(position)
    slot = np.asarray(slot)
    o0, _, _, _ = philox4x32(position, slot, np.full(np.broadcast(position, slot).shape, step & MASK),
                             np.full(np.broadcast(position, slot).shape, purpose),
                             seed & MASK, (seed >> 32) & MASK)
    return (o0 >> np.uint64(8)).astype(np.float64) * (2.0 ** -24)
