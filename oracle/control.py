"""Host-side control of the quantisation widths, written out plainly (test infrastructure).

Graph Extractor (SYLVIE guide, section 7).  Before training, the global in-degrees of all
boundary nodes are ranked and each node gets an importance factor p in [0, 1]: the node of
largest degree gets 1, the others their percentile position in the boundary-node pool, and equal
degrees give equal importance.  Reading used: p(v) is the fraction of boundary nodes whose degree
is at most deg(v) (the empirical percentile, kept as the exact fraction count / n).  The factor is
cut into as many mask levels as there are candidate widths: level = ceil(p * L) - 1 for L levels,
so the top quarter of the pool (for L = 4) gets the top level.  Relabelling nodes changes neither.

Quant Orchestrator (guide section 9, the worked example of Figure 7).  In each epoch the base
width b from the Coordinator and a node's level give the node's width: its level's candidate at
base 1 (1, 2, 4, 8 for levels 0..3) shifted up with the base, b * 2**level, clipped at the top
candidate 8.

Coordinator (guide section 8, Eq. 3 to 5, and the loop of section 11).  After epoch t: L_t is the
mean of the partitions' losses; F_t = lam * F_{t-1} + (1 - lam) * L_t, the first epoch starting the
average at L_0; LDR_t = (F_t - F_{t-1}) / et_t with et_t the epoch's time.  The next base width is
b_min after epoch 0; for t > delta it doubles (up to b_max) when LDR_t < LDR_{t-delta} and halves
(down to b_min) when LDR_t >= LDR_{t-delta}; otherwise it stays.  The execution mode of the next
epoch is synchronous in the first of those cases and asynchronous in the second, and unchanged
otherwise.  The guide's prose reads "LDR got worse" into the doubling branch while the formula's
LDR is negative when the loss falls; descent_magnitude=True takes the other reading by comparing
-LDR instead (doubling when the descent slowed).
"""
from __future__ import annotations

import numpy as np


def importance_counts(deg) -> np.ndarray:
    """For every node, how many nodes of the pool have a degree <= its own (p = count / n)."""
    deg = np.asarray(deg, dtype=np.int64)
    return np.searchsorted(np.sort(deg), deg, side="right").astype(np.int64)


def importance(deg) -> np.ndarray:
    deg = np.asarray(deg)
    return importance_counts(deg) / float(max(deg.size, 1))


def mask_levels(deg, n_levels: int = 4) -> np.ndarray:
    """ceil(p * L) - 1 with p = count / n, in integers."""
    deg = np.asarray(deg)
    n = deg.size
    cnt = importance_counts(deg)
    return ((cnt * n_levels + n - 1) // n - 1).astype(np.uint8)


def combine_and_clip(level, base_bits: int, max_bits: int = 8) -> np.ndarray:
    level = np.asarray(level, dtype=np.int64)
    return np.minimum(base_bits * (2 ** level), max_bits).astype(np.uint8)


class Coordinator:
    """The base width and execution mode after each epoch (Eq. 3 to 5), one call per epoch."""

    def __init__(self, lam: float = 0.9, delta: int = 5, b_min: int = 1, b_max: int = 8,
                 descent_magnitude: bool = False):
        self.lam = lam
        self.delta = delta
        self.b_min = b_min
        self.b_max = b_max
        self.sign = -1.0 if descent_magnitude else 1.0
        self.t = 0
        self.f_prev = None
        self.ldr = []             # LDR_0, LDR_1, ...
        self.bits = b_min         # the width epoch 0 runs at
        self.sync = True          # epoch 0 runs synchronously

    def step(self, partition_losses, epoch_time: float):
        """Record epoch t's losses and time; returns (base width, synchronous?) for epoch t + 1."""
        t = self.t
        l_t = sum(float(v) for v in partition_losses) / len(partition_losses)
        f_before = l_t if self.f_prev is None else self.f_prev
        f_t = self.lam * f_before + (1.0 - self.lam) * l_t
        ldr_t = self.sign * (f_t - f_before) / epoch_time
        self.ldr.append(ldr_t)
        if t == 0:
            self.bits = self.b_min
        elif t > self.delta:
            past = self.ldr[t - self.delta]
            if ldr_t < past:
                if self.bits < self.b_max:
                    self.bits = 2 * self.bits
                self.sync = True
            else:
                if self.bits > self.b_min:
                    self.bits = self.bits // 2
                self.sync = False
        self.f_prev = f_t
        self.t = t + 1
        return self.bits, self.sync
