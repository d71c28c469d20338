"""The seeded generator: determinism, exact sizes, the power-law tail and the width recipes."""
import numpy as np

from quantized_halo_aggregation_amd import synth


def test_deterministic_and_exact_sizes():
    wl = synth.WORKLOADS[1]
    a = synth.make_partition(wl)
    b = synth.make_partition(wl)
    for k in ("nbr_ptr", "nbr_idx", "deg", "mirror", "bits", "x", "grad_top"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    assert a.nbr_idx.size == wl.nnz
    assert a.nbr_ptr.dtype == np.int32 and a.nbr_idx.dtype == np.int32
    assert a.x.shape == (wl.n_in, wl.d) and a.x.dtype == np.float32
    assert a.weights[0].shape == (16, 16)
    # "halo bits drawn uniformly from {1,2,4,8}"
    counts = np.bincount(a.bits, minlength=9)[[1, 2, 4, 8]]
    assert counts.sum() == wl.n_h and counts.min() > wl.n_h / 4 - 4 * np.sqrt(wl.n_h)


def test_powerlaw_tail_exponent():
    """Discrete maximum-likelihood estimate (Clauset, Shalizi, Newman 2009) of the in-degree tail."""
    wl = synth.small_workload(60_000, 20_000, 1_500_000, 8, index=91)
    p = synth.make_partition(wl, with_features=False)
    deg = np.diff(p.nbr_ptr).astype(np.float64)
    xmin = 60.0
    tail = deg[(deg >= xmin) & (deg < 0.5 * deg.max())]
    alpha = 1.0 + tail.size / np.sum(np.log(tail / (xmin - 0.5)))
    assert abs(alpha - synth.ALPHA) < 0.15, alpha
    assert abs(deg.mean() - 25.0) < 1e-9


def test_top_fraction_width_recipe_includes_ties():
    rng = np.random.default_rng(0)
    deg = rng.integers(1, 20, size=1000)
    bits = synth.draw_bits(rng, ("top", 4, 8, 0.10), deg)
    hi = bits == 8
    assert hi.sum() >= 100
    assert deg[hi].min() >= deg[~hi].max() + 1 or deg[hi].min() > deg[~hi].max()
    t = np.sort(deg)[::-1][99]
    assert np.array_equal(hi, deg >= t)


def test_self_loop_insertion_keeps_rows_sorted():
    p = synth.make_partition(synth.WORKLOADS[1], with_features=False)
    ptr, idx = synth.with_self_loops(p.nbr_ptr, p.nbr_idx)
    assert idx.size == p.nbr_idx.size + p.n_in
    for v in range(0, p.n_in, 97):
        row = idx[ptr[v]:ptr[v + 1]]
        assert v in row and np.all(np.diff(row) > 0)
        assert np.array_equal(np.setdiff1d(row, [v]), p.nbr_idx[p.nbr_ptr[v]:p.nbr_ptr[v + 1]])
