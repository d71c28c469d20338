"""Philox4x32-10, written from Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
1, 2, 3" (SC'11), section on the Philox family.

State: a 128-bit counter (four 32-bit words c0..c3) and a 64-bit key (k0, k1).  One round multiplies
c0 and c2 by the two Philox-4x32 multipliers, keeping both halves of each 64-bit product, and
mixes the high halves with the other two counter words and the key; the key is bumped by the two
Weyl constants between rounds.  Ten rounds is the paper's recommended (crush-resistant with margin)
count.  Pure numpy, vectorised over arrays of counters; all arithmetic is done in uint64 and masked
to 32 bits.
"""
from __future__ import annotations

import numpy as np

MUL0 = 0xD2511F53
MUL1 = 0xCD9E8D57
WEYL0 = 0x9E3779B9
WEYL1 = 0xBB67AE85
ROUNDS = 10
_M32 = np.uint64(0xFFFFFFFF)


def _u64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.uint64) & _M32


def philox4x32(c0, c1, c2, c3, k0, k1, rounds: int = ROUNDS):
    """Return the four 32-bit output words (uint32 arrays) for the given counters and key."""
    c0, c1, c2, c3 = (_u64(c) for c in (c0, c1, c2, c3))
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    c0, c1, c2, c3 = (c.copy() for c in (c0, c1, c2, c3))
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for r in range(rounds):
        p0 = c0 * np.uint64(MUL0)            # < 2^64: exact in uint64
        p1 = c2 * np.uint64(MUL1)
        hi0, lo0 = p0 >> np.uint64(32), p0 & _M32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _M32
        n0 = hi1 ^ c1 ^ np.uint64(k0)
        n1 = lo1
        n2 = hi0 ^ c3 ^ np.uint64(k1)
        n3 = lo0
        c0, c1, c2, c3 = n0, n1, n2, n3
        if r + 1 < rounds:
            k0 = (k0 + WEYL0) & 0xFFFFFFFF
            k1 = (k1 + WEYL1) & 0xFFFFFFFF
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def rounding_thresholds(node_ids, n_features: int, seed: int, epoch: int, stream_id: int) -> np.ndarray:
    """16-bit uniform thresholds u[r, j] for stochastic rounding of feature j of node ``node_ids[r]``.

    Counter = (node id, j // 8, epoch, stream id); key = (low, high) 32-bit halves of ``seed``.
    One generator call serves eight consecutive features: feature 8g + i takes word i // 2 of call g,
    its low half when i is even and its high half when i is odd.
    """
    node_ids = np.asarray(node_ids, dtype=np.uint64)
    n_groups = (n_features + 7) // 8
    grp = np.arange(n_groups, dtype=np.uint64)
    c0 = node_ids[:, None] + np.zeros((1, n_groups), np.uint64)
    c1 = np.zeros_like(c0) + grp[None, :]
    w = philox4x32(c0, c1, np.uint64(epoch), np.uint64(stream_id), seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    words = np.stack(w, axis=-1)                        # [n, groups, 4] uint32
    lo = words & np.uint32(0xFFFF)
    hi = words >> np.uint32(16)
    halves = np.stack([lo, hi], axis=-1).reshape(node_ids.size, n_groups * 8)   # feature order
    return halves[:, :n_features].astype(np.uint32)
