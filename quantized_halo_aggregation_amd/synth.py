"""Seeded synthetic partitions: the only module that both the HIP path and the oracle consume.

It builds inputs and nothing else -- no normalisation, quantisation, aggregation or projection
arithmetic lives here.  Every array is drawn from numpy's PCG64 with a fixed seed, so a config
and a seed always give the same partition on any host.

What one partition holds (SYLVIE guide, sections 3 and 7: a GPU owns its inner nodes; its halo
(boundary) nodes are remote neighbours whose importance proxy is their *global* in-degree):

* ``nbr_ptr``/``nbr_idx`` -- int32 CSR of the neighbour lists N(v) of the ``n_in`` inner rows,
  no self-loops, columns ascending.  Column ids ``< n_in`` are inner nodes, ids ``n_in + k`` are
  halo node k, so every row lists its inner neighbours first.
* ``deg`` -- int32 global in-degree of every column node (inner and halo).
* ``mirror`` -- int32, halo k is the remote copy of inner node ``mirror[k]`` (the one-GPU stand-in
  for the partition that owns it).
* ``bits`` -- uint8 per-halo bit width.  Halo nodes are numbered by width, widest first, so equal
  widths are contiguous (``number_halos_by_width``).
* ``x`` -- float32 [n_in, d] layer-1 embeddings ~ N(0, 1); ``weights`` -- per-layer W ~ N(0, 1/fan_in);
  ``grad_top`` -- float32 upstream gradient ~ N(0, 1).

Graph recipe: inner in-degrees follow a discrete power law ``floor(k_min * U^(-1/(alpha-1)))``
clipped to ``[1, k_max]`` with alpha = 2.1, ``k_min`` fitted by bisection to the target mean and
a seeded +-1 adjustment to hit the exact edge count.  Row v then draws ``deg_v`` distinct sources
from all other column nodes with probability proportional to their degree (a Chung-Lu style
preferential model), by repeated draws with de-duplication, or by weighted sampling without
replacement (exponential keys) for rows that take more than 2% of all columns.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

ALPHA = 2.1

# seeds: graph 1000+i, features 2000+i, weights 3000+i, bits 4000+i for workload i
QUANT_SEED = 0x5EED5EED5EED5EED


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic partition recipe (sizes follow the five partitions the method is measured on)."""
    index: int
    name: str
    n_in: int
    n_h: int
    nnz: int            # directed neighbour edges, self-loops excluded
    d: int              # hidden width of every layer
    layers: int
    model: str          # "gcn" or "sage"
    bits: tuple         # ("uniform", choices) | ("top", base, high, frac) | ("const", b)
    k_max: int | None = None

    @property
    def n_cols(self) -> int:
        return self.n_in + self.n_h

    def describe(self) -> str:
        return (f"{self.name}: {self.n_in} inner + {self.n_h} halo nodes, ~{self.nnz} edges, "
                f"d={self.d}, {self.layers} {self.model.upper()} layer(s)")


WORKLOADS = {
    1: Workload(1, "tiny-partition", 2048, 512, 20_000, 16, 1, "gcn", ("uniform", (1, 2, 4, 8))),
    2: Workload(2, "gcn-300k-d128", 300_000, 150_000, 7_500_000, 128, 1, "gcn", ("top", 4, 8, 0.10)),
    3: Workload(3, "dense-degree-30k-d256", 30_000, 60_000, 14_700_000, 256, 4, "gcn",
                ("top", 2, 4, 0.20), k_max=20_000),
    4: Workload(4, "sage-mean-600k-d256", 600_000, 300_000, 12_000_000, 256, 4, "sage", ("const", 1)),
    5: Workload(5, "gcn-2.4m-d128", 1_800_000, 600_000, 62_000_000, 128, 8, "gcn", ("const", 4)),
}


def small_workload(n_in: int, n_h: int, nnz: int, d: int, bits=("uniform", (1, 2, 4, 8, 32)),
                   model: str = "gcn", k_max: int | None = None, index: int = 90) -> Workload:
    """An ad-hoc partition for parity tests that must finish in seconds on the CPU."""
    return Workload(index, f"small-{n_in}-{n_h}-{d}", n_in, n_h, nnz, d, 1, model, bits, k_max)


# --------------------------------------------------------------------------------------------
# degree sequence
# --------------------------------------------------------------------------------------------

def powerlaw_degrees(rng: np.random.Generator, n: int, total: int, k_max: int,
                     alpha: float = ALPHA) -> np.ndarray:
    """Integer degrees with a power-law tail, clipped to [1, k_max], summing exactly to ``total``."""
    u = rng.random(n)
    tail = u ** (-1.0 / (alpha - 1.0))

    def draw(k_min: float) -> np.ndarray:
        return np.clip(np.floor(k_min * tail), 1, k_max).astype(np.int64)

    target_mean = total / n
    lo, hi = 1e-3, max(2.0, 4.0 * target_mean)
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if draw(mid).mean() < target_mean:
            lo = mid
        else:
            hi = mid
    deg = draw(hi)
    diff = int(total - deg.sum())
    if diff > 0:
        cand = np.flatnonzero(deg < k_max)
        pick = rng.choice(cand, size=min(diff, cand.size), replace=False)
        deg[pick] += 1
    elif diff < 0:
        cand = np.flatnonzero(deg > 1)
        pick = rng.choice(cand, size=min(-diff, cand.size), replace=False)
        deg[pick] -= 1
    return deg


# --------------------------------------------------------------------------------------------
# neighbour sampling
# --------------------------------------------------------------------------------------------

def _dedupe(keys: np.ndarray) -> np.ndarray:
    return np.unique(keys)


def sample_neighbours(rng: np.random.Generator, want: np.ndarray, weight: np.ndarray,
                      heavy_frac: float = 0.02, max_rounds: int = 40):
    """Row v draws ``want[v]`` distinct columns != v with probability proportional to ``weight``.

    Returns (ptr, idx) int32 CSR with columns ascending.  Rows whose demand cannot be met after
    ``max_rounds`` top-up rounds (only possible for extreme weight concentration) keep what they got.
    """
    n_rows = want.size
    n_cols = weight.size
    w = weight.astype(np.float64)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]

    heavy = np.flatnonzero(want > heavy_frac * n_cols)
    light_want = want.copy()
    light_want[heavy] = 0

    keys_parts = []
    # light rows: draw with replacement, drop self-loops and duplicates, top up the shortfall
    need = light_want.copy()
    have_keys = np.empty(0, dtype=np.int64)
    for _ in range(max_rounds):
        total = int(need.sum())
        if total == 0:
            break
        rows = np.repeat(np.arange(n_rows, dtype=np.int64), need)
        cols = np.searchsorted(cdf, rng.random(total), side="right").astype(np.int64)
        cols = np.minimum(cols, n_cols - 1)
        keep = cols != rows
        new = rows[keep] * n_cols + cols[keep]
        if have_keys.size:
            # merge only the rows that were short
            short_rows = need > 0
            owner = have_keys // n_cols
            sel = short_rows[owner]
            merged = _dedupe(np.concatenate([have_keys[sel], new]))
            have_keys = np.concatenate([have_keys[~sel], merged])
        else:
            have_keys = _dedupe(new)
        got = np.bincount(have_keys // n_cols, minlength=n_rows)
        # trim rows that overshot (cannot happen with exact draws, kept for safety)
        need = np.maximum(light_want - got, 0)
    keys_parts.append(have_keys)

    # heavy rows: weighted sampling without replacement with exponential keys
    for v in heavy:
        k = int(min(want[v], n_cols - 1))
        e = rng.exponential(size=n_cols) / np.maximum(w, 1e-300)
        e[v] = np.inf
        chosen = np.argpartition(e, k - 1)[:k]
        keys_parts.append(np.int64(v) * n_cols + chosen.astype(np.int64))

    keys = np.sort(np.concatenate(keys_parts))
    rows = keys // n_cols
    idx = (keys - rows * n_cols).astype(np.int32)
    counts = np.bincount(rows, minlength=n_rows)
    ptr = np.zeros(n_rows + 1, dtype=np.int64)
    np.cumsum(counts, out=ptr[1:])
    return ptr.astype(np.int32), idx


# --------------------------------------------------------------------------------------------
# a whole partition
# --------------------------------------------------------------------------------------------

@dataclasses.dataclass
class Partition:
    wl: Workload
    nbr_ptr: np.ndarray
    nbr_idx: np.ndarray
    deg: np.ndarray
    mirror: np.ndarray
    bits: np.ndarray
    x: np.ndarray
    weights: list
    grad_top: np.ndarray

    @property
    def n_in(self):
        return self.wl.n_in

    @property
    def n_h(self):
        return self.wl.n_h

    @property
    def d(self):
        return self.wl.d

    @property
    def nnz(self):
        return int(self.nbr_idx.size)

    def stats(self) -> dict:
        rl = np.diff(self.nbr_ptr)
        halo_edges = int((self.nbr_idx >= self.n_in).sum())
        return {"nnz": self.nnz, "mean_row": float(rl.mean()), "max_row": int(rl.max()),
                "halo_edges": halo_edges,
                "bits_hist": {int(b): int((self.bits == b).sum()) for b in np.unique(self.bits)}}


def draw_bits(rng: np.random.Generator, recipe: tuple, halo_deg: np.ndarray) -> np.ndarray:
    """Per-halo widths.  ("top", base, high, frac): halos whose degree is at least that of the
    ceil(frac * n_h)-th largest get ``high`` (so equal degrees get equal widths)."""
    n_h = halo_deg.size
    kind = recipe[0]
    if kind == "uniform":
        return rng.choice(np.asarray(recipe[1], dtype=np.uint8), size=n_h)
    if kind == "const":
        return np.full(n_h, recipe[1], dtype=np.uint8)
    if kind == "top":
        _, base, high, frac = recipe
        if n_h == 0:
            return np.zeros(0, dtype=np.uint8)
        m = max(1, int(math.ceil(frac * n_h)))
        t = np.sort(halo_deg)[::-1][m - 1]
        return np.where(halo_deg >= t, high, base).astype(np.uint8)
    raise ValueError(f"unknown bits recipe {recipe!r}")


def number_halos_by_width(n_in, ptr, idx, deg, mirror, bits):
    """Renumbers the halo nodes so that equal widths are contiguous, widest first (a stable order
    otherwise).  This is a relabelling only: the receiver is free to number its halo nodes, and
    doing it by width lets a width-grouped packed buffer be addressed by arithmetic."""
    n_h = bits.size
    perm = np.argsort(-bits.astype(np.int64), kind="stable")          # new halo id -> old halo id
    if np.array_equal(perm, np.arange(n_h)):
        return ptr, idx, deg, mirror, bits
    inv = np.empty(n_h, dtype=np.int64)
    inv[perm] = np.arange(n_h)
    n_rows = ptr.size - 1
    n_cols = n_in + n_h
    cols = idx.astype(np.int64)
    halo = cols >= n_in
    cols[halo] = n_in + inv[cols[halo] - n_in]
    rows = np.repeat(np.arange(n_rows, dtype=np.int64), np.diff(ptr))
    keys = np.sort(rows * n_cols + cols)
    new_idx = (keys - (keys // n_cols) * n_cols).astype(np.int32)
    new_deg = np.concatenate([deg[:n_in], deg[n_in:][perm]]).astype(np.int32)
    return ptr, new_idx, new_deg, mirror[perm], bits[perm]


def make_partition(wl: Workload, bits_override=None, with_features: bool = True) -> Partition:
    g = np.random.default_rng(1000 + wl.index)
    k_max = wl.k_max
    if k_max is None:
        k_max = int(100 * wl.nnz / wl.n_in)
    k_max = min(k_max, wl.n_cols - 1)
    want = powerlaw_degrees(g, wl.n_in, wl.nnz, k_max)
    if wl.n_h <= wl.n_in:
        mirror = g.choice(wl.n_in, size=wl.n_h, replace=False).astype(np.int32)
    else:
        mirror = g.integers(0, wl.n_in, size=wl.n_h).astype(np.int32)
    weight = np.concatenate([want, want[mirror]]).astype(np.float64)
    ptr, idx = sample_neighbours(g, want, weight)
    row_len = np.diff(ptr).astype(np.int32)
    deg = np.concatenate([row_len, row_len[mirror]]).astype(np.int32)

    recipe = bits_override if bits_override is not None else wl.bits
    bits = draw_bits(np.random.default_rng(4000 + wl.index), recipe, deg[wl.n_in:])
    ptr, idx, deg, mirror, bits = number_halos_by_width(wl.n_in, ptr, idx, deg, mirror, bits)

    x = np.zeros((0, wl.d), np.float32)
    weights = []
    grad_top = np.zeros((0, wl.d), np.float32)
    if with_features:
        f = np.random.default_rng(2000 + wl.index)
        x = f.standard_normal((wl.n_in, wl.d), dtype=np.float32)
        grad_top = f.standard_normal((wl.n_in, wl.d), dtype=np.float32)
        wr = np.random.default_rng(3000 + wl.index)
        fan_in = 2 * wl.d if wl.model == "sage" else wl.d
        for _ in range(wl.layers):
            weights.append((wr.standard_normal((wl.d, fan_in)) / math.sqrt(fan_in)).astype(np.float32))
    return Partition(wl, ptr, idx, deg, mirror, bits, x, weights, grad_top)


# --------------------------------------------------------------------------------------------
# plain data-structure views (no arithmetic on values)
# --------------------------------------------------------------------------------------------

def with_self_loops(ptr: np.ndarray, idx: np.ndarray):
    """Insert column v into row v of a CSR whose rows are sorted and hold no self-loop."""
    n = ptr.size - 1
    rows = np.repeat(np.arange(n, dtype=np.int64), np.diff(ptr))
    # position of v inside row v = number of columns < v in that row
    before = np.bincount(rows[idx < rows], minlength=n)
    at = ptr[:-1].astype(np.int64) + before
    new_idx = np.insert(idx, at, np.arange(n, dtype=np.int32)).astype(np.int32)
    new_ptr = (ptr.astype(np.int64) + np.arange(n + 1)).astype(np.int32)
    return new_ptr, new_idx


def halo_rows(part: Partition, x_inner: np.ndarray) -> np.ndarray:
    """Mirror model send set: the embeddings of the inner nodes that play the halo nodes."""
    return x_inner[part.mirror]
