"""Pins of the oracle's Graph Extractor, Quant Orchestrator and Coordinator (oracle/control.py)."""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import control as OC

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fig7_node_bits.txt")


def read_fig7():
    """(mask widths, [(base, expected widths)]) from the guide's Figure 7 fixture."""
    mask, cases = None, []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            if line.startswith("mask"):
                mask = [int(v) for v in line.split()[1:]]
            else:
                left, right = line.split("->")
                cases.append((int(left.split()[1]), [int(v) for v in right.split()]))
    return mask, cases


def test_figure7_widths_follow_from_mask_and_base():
    mask, cases = read_fig7()
    assert len(cases) == 3
    level = np.log2(mask).astype(int)          # the mask as levels: width at base 1 is 2**level
    for base, want in cases:
        assert OC.combine_and_clip(level, base).tolist() == want, base


def test_importance_on_a_worked_example():
    # degrees 5, 1, 5, 3, 9: sorted 1, 3, 5, 5, 9, so at most each degree sit 4, 1, 4, 2, 5 nodes
    deg = [5, 1, 5, 3, 9]
    assert OC.importance(deg).tolist() == [0.8, 0.2, 0.8, 0.4, 1.0]
    # ceil(p * 4) - 1: 3.2 -> 3, 0.8 -> 0, 1.6 -> 1, 4 -> 3
    assert OC.mask_levels(deg).tolist() == [3, 0, 3, 1, 3]


def test_importance_properties():
    """Guide section 16: the largest degree gets 1, equal degrees equal importance, relabelling the
    nodes does not change a node's importance; and importance never falls as degree rises."""
    rng = np.random.default_rng(0)
    deg = rng.integers(1, 50, size=997)
    p = OC.importance(deg)
    assert np.all(p[deg == deg.max()] == 1.0)
    for d in np.unique(deg):
        assert np.unique(p[deg == d]).size == 1
    perm = rng.permutation(deg.size)
    assert np.array_equal(OC.importance(deg[perm]), p[perm])
    order = np.argsort(deg, kind="stable")
    assert np.all(np.diff(p[order]) >= 0)


def test_levels_against_exact_fractions():
    rng = np.random.default_rng(1)
    for n, L in ((1, 4), (7, 4), (100, 4), (333, 3), (64, 8)):
        deg = rng.integers(0, 20, size=n)
        want = []
        for v in deg:
            p = Fraction(int((deg <= v).sum()), n)
            k = -(-(p * L).numerator // (p * L).denominator)      # ceil of a fraction
            want.append(k - 1)
        assert OC.mask_levels(deg, L).tolist() == want
        lv = OC.mask_levels(deg, L)
        assert lv.min() >= 0 and lv.max() == L - 1


def test_combine_and_clip_covers_every_base():
    level = np.arange(4)
    assert OC.combine_and_clip(level, 1).tolist() == [1, 2, 4, 8]
    assert OC.combine_and_clip(level, 2).tolist() == [2, 4, 8, 8]
    assert OC.combine_and_clip(level, 4).tolist() == [4, 8, 8, 8]
    assert OC.combine_and_clip(level, 8).tolist() == [8, 8, 8, 8]
    # widths never increase along a numbering by descending level, whatever the base
    lv = np.sort(np.random.default_rng(2).integers(0, 4, 50))[::-1]
    for b in (1, 2, 4, 8):
        assert np.all(np.diff(OC.combine_and_clip(lv, b).astype(int)) <= 0)


# A hand-worked trace of Eq. 3-5 with lam = 0 (so F_t = L_t), delta = 2, one partition, unit epoch
# times: losses 10, 9, 8, 6, 3, 2.5, 2.4, 2.4 give LDR 0, -1, -1, -2, -3, -0.5, -0.1, 0.
TRACE = [10, 9, 8, 6, 3, 2.5, 2.4, 2.4]
# after epoch t: (base width, synchronous) of epoch t + 1
LITERAL = [(1, True), (1, True), (1, True),      # t <= delta: unchanged from the start
           (2, True),                            # -2 < -1: double, synchronous
           (4, True),                            # -3 < -1: double
           (2, False),                           # -0.5 >= -2: halve, asynchronous
           (1, False),                           # -0.1 >= -3: halve
           (1, False)]                           # 0 >= -0.5: already at b_min
MAGNITUDE = [(1, True), (1, True), (1, True),    # comparing -LDR: 2, 3, 0.5, 0.1, 0 against 1, 1, 2, 3, 0.5
             (1, False), (1, False),
             (2, True), (4, True), (8, True)]


@pytest.mark.parametrize("descent_magnitude,want", [(False, LITERAL), (True, MAGNITUDE)])
def test_coordinator_hand_trace(descent_magnitude, want):
    c = OC.Coordinator(lam=0.0, delta=2, descent_magnitude=descent_magnitude)
    got = [c.step([v], 1.0) for v in TRACE]
    assert got == want
    assert np.allclose(c.ldr, [0, -1, -1, -2, -3, -0.5, -0.1, 0] if not descent_magnitude
                       else [0, 1, 1, 2, 3, 0.5, 0.1, 0])


def test_coordinator_smoothing_partitions_and_bounds():
    # lam = 0.5, two partitions: L_t is their mean, F_0 = L_0, then F_t = (F_{t-1} + L_t) / 2
    c = OC.Coordinator(lam=0.5, delta=1)
    c.step([100.0, 100.0], 2.0)
    c.step([50.0, 70.0], 2.0)             # L = 60, F = 80, LDR = -10
    assert c.f_prev == 80.0 and c.ldr[-1] == -10.0
    # an ever faster descent doubles the width up to b_max and stays there, synchronously
    c = OC.Coordinator(lam=0.0, delta=1)
    loss, out = 1000.0, []
    for t in range(10):
        loss -= 2.0 ** t
        out.append(c.step([loss], 1.0))
    assert [b for b, _ in out] == [1, 1, 2, 4, 8, 8, 8, 8, 8, 8]
    assert all(s for _, s in out)
    # a flat loss halves down to b_min and runs asynchronously after delta epochs
    c = OC.Coordinator(lam=0.9, delta=3)
    out = [c.step([1.0, 3.0], 0.5) for _ in range(8)]
    assert out[:4] == [(1, True)] * 4 and out[4:] == [(1, False)] * 4
