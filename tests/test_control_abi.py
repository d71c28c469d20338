"""The library's host-side width control (qha_mask_levels, qha_node_bits, qha_level_order,
qha_coordinator_*) against the oracle and the guide's Figure 7 example.  CPU only."""
import numpy as np
import pytest

from oracle import control as OC
from test_oracle_control import LITERAL, MAGNITUDE, TRACE, read_fig7


@pytest.fixture(scope="module")
def B():
    from quantized_halo_aggregation_amd import binding
    return binding


def test_figure7_through_the_library(B):
    mask, cases = read_fig7()
    level = np.log2(mask).astype(np.uint8)
    for base, want in cases:
        assert B.node_bits(level, base).tolist() == want


@pytest.mark.parametrize("n,L", [(1, 4), (5, 4), (1000, 4), (4097, 3), (300, 8), (150000, 4)])
def test_mask_levels_match_the_oracle(B, n, L):
    rng = np.random.default_rng(n + L)
    deg = rng.integers(1, 3000, size=n).astype(np.int32) if n > 5 else np.array([5, 1, 5, 3, 9][:n], np.int32)
    level, imp = B.mask_levels(deg, L)
    assert np.array_equal(level, OC.mask_levels(deg, L))
    assert np.array_equal(imp, OC.importance(deg))


def test_node_bits_and_level_order(B):
    rng = np.random.default_rng(3)
    level = rng.integers(0, 4, size=2000).astype(np.uint8)
    for base in (1, 2, 4, 8):
        assert np.array_equal(B.node_bits(level, base), OC.combine_and_clip(level, base))
    order = B.level_order(level)
    assert np.array_equal(order, np.argsort(-level.astype(int), kind="stable"))
    for base in (1, 2, 4, 8):          # widths never increase along the numbering
        bits = B.node_bits(level[order], base)
        assert np.all(np.diff(bits.astype(int)) <= 0)
        assert B.pack_classes(bits, 128) is not None
    with pytest.raises(Exception):
        B.node_bits(np.array([8], np.uint8), 1)
    with pytest.raises(Exception):
        B.node_bits(level, 3)
    with pytest.raises(Exception):
        B.mask_levels(np.array([1, 2], np.int32), 0)


@pytest.mark.parametrize("descent_magnitude,want", [(False, LITERAL), (True, MAGNITUDE)])
def test_coordinator_hand_trace(B, descent_magnitude, want):
    c = B.Coordinator(lam=0.0, delta=2, descent_magnitude=descent_magnitude)
    assert [c.step([v], 1.0) for v in TRACE] == want


def test_coordinator_matches_the_oracle_on_random_traces(B):
    rng = np.random.default_rng(11)
    for trial in range(40):
        lam = float(rng.choice([0.0, 0.5, 0.9, 1.0]))
        delta = int(rng.integers(1, 12))
        b_min, b_max = (1, 8) if trial % 3 else (2, 4)
        mag = bool(trial % 2)
        n_part = int(rng.integers(1, 9))
        ref = OC.Coordinator(lam=lam, delta=delta, b_min=b_min, b_max=b_max, descent_magnitude=mag)
        lib = B.Coordinator(lam=lam, delta=delta, b_min=b_min, b_max=b_max, descent_magnitude=mag)
        loss = 5.0 + rng.random(n_part)
        for t in range(60):
            loss = np.maximum(loss * (0.9 + 0.15 * rng.random(n_part)) + 0.05 * rng.standard_normal(n_part), 0.01)
            et = float(0.2 + rng.random())
            assert lib.step(loss, et) == ref.step(loss.tolist(), et), (trial, t)
        assert lib.state.last_ldr == ref.ldr[-1]


def test_coordinator_rejects_bad_arguments(B):
    with pytest.raises(Exception):
        B.Coordinator(lam=1.5)
    with pytest.raises(Exception):
        B.Coordinator(delta=0)
    with pytest.raises(Exception):
        B.Coordinator(b_min=3)
    with pytest.raises(Exception):
        B.Coordinator(b_min=8, b_max=4)
    c = B.Coordinator()
    with pytest.raises(Exception):
        c.step([], 1.0)
    with pytest.raises(Exception):
        c.step([1.0], 0.0)
