"""Property tests of the library's host helpers on random inputs (CPU): the aggregation plan, the
packed-message layouts and the CSR transpose.  Each property is the helper's documented contract in
include/qha.h, checked by plain numpy arithmetic."""
import ctypes as C

import numpy as np
from hypothesis import given, settings, strategies as st

from quantized_halo_aggregation_amd import binding as B

SETTINGS = settings(max_examples=150, deadline=None)


def plan_host(lens, chunk, group_edges, skip_empty):
    ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pl = B.AggPlanStruct()
    B._check(B._plan_size(ptr.size - 1, ptr.ctypes.data, chunk, group_edges, int(skip_empty), C.byref(pl)), "size")
    items = np.zeros(4 * max(pl.n_items, 1), np.int32)
    split_row = np.zeros(max(pl.n_split_rows, 1), np.int32)
    split_ptr = np.zeros(pl.n_split_rows + 1, np.int32)
    B._check(B._plan_fill(ptr.ctypes.data, C.byref(pl), items.ctypes.data, split_row.ctypes.data,
                          split_ptr.ctypes.data), "fill")
    return ptr, pl, items[:4 * pl.n_items].reshape(-1, 4), split_row[:pl.n_split_rows], split_ptr


@SETTINGS
@given(lens=st.lists(st.one_of(st.integers(0, 3), st.integers(0, 40), st.integers(0, 1500)), max_size=120),
       chunk=st.sampled_from([1, 2, 7, 64, 256, 512]), group_edges=st.sampled_from([1, 8, 128, 256]),
       skip_empty=st.booleans())
def test_plan_contract(lens, chunk, group_edges, skip_empty):
    lens = np.asarray(lens, np.int64)
    ptr, pl, items, split_row, split_ptr = plan_host(lens, chunk, group_edges, skip_empty)
    n = lens.size
    split = lens > chunk
    # split rows, ascending, and their chunks first, in order, each at most `chunk` edges
    assert list(split_row) == list(np.flatnonzero(split))
    assert pl.n_split_rows == split.sum() and split_ptr[0] == 0
    assert pl.n_split_items == split_ptr[-1] == sum(-(-int(x) // chunk) for x in lens[split])
    for m, r in enumerate(split_row):
        ch = items[split_ptr[m]:split_ptr[m + 1]]
        assert (ch[:, 0] == r).all() and (ch[:, 1] == 1).all()
        assert ch[0, 2] == ptr[r] and ch[-1, 3] == ptr[r + 1] and (ch[1:, 2] == ch[:-1, 3]).all()
        assert ((ch[:, 3] - ch[:, 2]) <= chunk).all() and ((ch[:, 3] - ch[:, 2]) > 0).all()
    # the other items: runs of whole consecutive rows
    seen = np.zeros(n, np.int64)
    for r0, nr, e0, e1 in items[pl.n_split_items:]:
        assert 1 <= nr <= B.GROUP_ROWS
        assert e0 == ptr[r0] and e1 == ptr[r0 + nr]
        g = lens[r0:r0 + nr]
        assert not (g > chunk).any()
        if nr > 1:
            assert (g > 0).all() and g.sum() <= group_edges
        seen[r0:r0 + nr] += 1
    want = np.where(split, 0, np.where(lens == 0, 0 if skip_empty else 1, 1))
    assert np.array_equal(seen, want)
    # every edge exactly once
    cover = np.zeros(int(ptr[-1]), np.int64)
    for r0, nr, e0, e1 in items:
        cover[e0:e1] += 1
    assert (cover == 1).all()
    assert B._plan_ws(C.byref(pl), 64) == pl.n_split_items * 64 * 8


widths = st.sampled_from([1, 2, 4, 8, 32])


@SETTINGS
@given(runs=st.lists(st.tuples(widths, st.integers(1, 40)), min_size=1, max_size=12),
       d=st.sampled_from([16, 32, 64, 128, 256, 512]))
def test_width_classes_give_the_per_row_layout(runs, d):
    bits = np.concatenate([np.full(c, b, np.uint8) for b, c in runs])
    off, total = B.pack_layout(bits, d)
    words = np.where(bits == 32, d, (d * bits.astype(np.int64) + 31) // 32)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(words)]).astype(np.uint32)) and total == words.sum()
    n_runs = 1 + int((bits[1:] != bits[:-1]).sum())
    cls = B.pack_classes(bits, d)
    if n_runs > 8:
        assert cls is None
        return
    assert cls is not None and cls.n == n_runs and cls.start[cls.n] == bits.size
    for c in range(cls.n):
        rows = np.arange(cls.start[c], cls.start[c + 1])
        assert (bits[rows] == cls.bits[c]).all()
        w = d if cls.bits[c] == 32 else (d * cls.bits[c] + 31) // 32
        assert np.array_equal(cls.base[c] + (rows - cls.start[c]) * w, off[rows])


@SETTINGS
@given(st.data())
def test_csr_transpose_round_trip(data):
    n_rows = data.draw(st.integers(0, 60))
    n_cols = data.draw(st.integers(1, 60))
    rows = [sorted(data.draw(st.sets(st.integers(0, n_cols - 1), max_size=min(n_cols, 20)))) for _ in range(n_rows)]
    ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    idx = np.array([c for r in rows for c in r], np.int32)
    B.validate_csr(ptr, idx, n_cols)
    colptr, rowidx = B.csr_transpose(ptr, idx, n_cols)
    assert np.array_equal(np.diff(colptr), np.bincount(idx, minlength=n_cols))
    B.validate_csr(colptr, rowidx, n_rows if n_rows else 1)        # rows ascending within each column
    back_ptr, back_idx = B.csr_transpose(colptr, rowidx, n_rows)
    assert np.array_equal(back_ptr, ptr) and np.array_equal(back_idx, idx)
