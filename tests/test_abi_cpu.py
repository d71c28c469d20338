"""The C ABI without a GPU: the library loads, exports every entry point of include/qha.h, its host
helpers compute the documented layouts, and bad arguments are rejected before any HIP call.

Argument-error cases pass fake (never dereferenced) device addresses: the checks must fire first.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from quantized_halo_aggregation_amd import binding as B

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qha.h")
FAKE = 0x10000          # 16-byte aligned, never dereferenced by a call that fails its checks


def test_header_symbols_are_exported():
    text = open(HDR).read()
    declared = set(re.findall(r"\b(qha_[a-z0-9_]+)\s*\(", text))
    assert declared, "no declarations found"
    lib = C.CDLL(B.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared in qha.h but not exported"
    assert declared == set(B.EXPORTED)
    assert B.abi_version() == 3


def test_status_strings():
    assert B._status_string(0) == b"ok"
    assert B._status_string(2) == b"unsupported"


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256, 512])
def test_pack_layout(d):
    bits = np.array([1, 2, 4, 8, 32, 4, 1], np.uint8)
    off, total = B.pack_layout(bits, d)
    sizes = [d if b == 32 else (d * int(b) + 31) // 32 for b in bits]
    assert list(off) == [0] + list(np.cumsum(sizes))
    assert total == sum(sizes)


def test_pack_classes_describe_the_same_layout():
    d = 128
    bits = np.array([8] * 5 + [4] * 7 + [32] * 2 + [1] * 3, np.uint8)
    off, total = B.pack_layout(bits, d)
    cl = B.pack_classes(bits, d)
    assert cl.n == 4
    assert list(cl.bits[:4]) == [8, 4, 32, 1] and list(cl.start[:5]) == [0, 5, 12, 14, 17]
    for r in range(bits.size):
        c = max(i for i in range(cl.n) if cl.start[i] <= r)
        w = d if cl.bits[c] == 32 else d * cl.bits[c] // 32
        assert cl.base[c] + (r - cl.start[c]) * w == off[r]
    # too many runs: the per-row table is needed
    assert B.pack_classes(np.array([1, 2] * 5, np.uint8), d) is None
    assert B.pack_classes(np.zeros(0, np.uint8), d).n == 1


def test_pack_layout_rejects_bad_width_and_d():
    with pytest.raises(ValueError, match="not in"):
        B.pack_layout(np.array([4, 3], np.uint8), 128)
    with pytest.raises(ValueError, match="not supported"):
        B.pack_layout(np.array([4], np.uint8), 24)


def test_csr_transpose_and_validate():
    rng = np.random.default_rng(0)
    n_rows, n_cols = 50, 70
    dense = rng.random((n_rows, n_cols)) < 0.1
    ptr = np.concatenate([[0], np.cumsum(dense.sum(1))]).astype(np.int32)
    idx = np.nonzero(dense)[1].astype(np.int32)
    B.validate_csr(ptr, idx, n_cols)
    cptr, ridx = B.csr_transpose(ptr, idx, n_cols)
    dt = dense.T
    assert np.array_equal(cptr, np.concatenate([[0], np.cumsum(dt.sum(1))]))
    assert np.array_equal(ridx, np.nonzero(dt)[1])
    bad = idx.copy()
    bad[3] = n_cols
    with pytest.raises(ValueError, match="outside"):
        B.validate_csr(ptr, bad, n_cols)
    unsorted = idx.copy()
    r = int(np.argmax(np.diff(ptr) >= 2))
    unsorted[ptr[r]], unsorted[ptr[r] + 1] = unsorted[ptr[r] + 1], unsorted[ptr[r]]
    with pytest.raises(ValueError, match="ascending"):
        B.validate_csr(ptr, unsorted, n_cols)


def _plan_host(ptr, chunk, skip_empty, group_edges=256):
    st = B.AggPlanStruct()
    B._check(B._plan_size(ptr.size - 1, ptr.ctypes.data, chunk, group_edges, int(skip_empty), C.byref(st)), "size")
    items = np.zeros(4 * max(st.n_items, 1), np.int32)
    split_row = np.zeros(max(st.n_split_rows, 1), np.int32)
    sp = np.zeros(st.n_split_rows + 1, np.int32)
    B._check(B._plan_fill(ptr.ctypes.data, C.byref(st), items.ctypes.data, split_row.ctypes.data, sp.ctypes.data),
             "fill")
    return st, items[:4 * st.n_items].reshape(-1, 4), split_row[:st.n_split_rows], sp


@pytest.mark.parametrize("skip_empty", [False, True])
@pytest.mark.parametrize("group_edges", [1, 8, 256])
def test_agg_plan_covers_every_edge_and_row_once(skip_empty, group_edges):
    lens = np.array([0, 3, 1200, 5, 0, 512, 513, 2000, 1, 2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 7, 0],
                    np.int32)
    ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    chunk = 512
    st, items, split_row, split_ptr = _plan_host(ptr, chunk, skip_empty, group_edges)
    edge_cover = np.zeros(ptr[-1], np.int32)
    row_cover = np.zeros(lens.size, np.int32)
    for it, (r0, nr, e0, e1) in enumerate(items):
        assert nr >= 1 and nr <= B.GROUP_ROWS
        edge_cover[e0:e1] += 1
        if it < st.n_split_items:
            assert nr == 1 and lens[r0] > chunk and e1 - e0 <= chunk
        else:
            # a group is a run of whole consecutive rows; empty rows stand alone
            assert e0 == ptr[r0] and e1 == ptr[r0 + nr]
            row_cover[r0:r0 + nr] += 1
            if nr > 1:
                assert (lens[r0:r0 + nr] > 0).all() and e1 - e0 <= max(group_edges, lens[r0:r0 + nr].max())
    assert (edge_cover == 1).all()
    split = lens > chunk
    assert (row_cover[split] == 0).all()
    want = np.where(split, 0, np.where(lens == 0, 0 if skip_empty else 1, 1))
    assert np.array_equal(row_cover, want)
    assert list(split_row) == [2, 6, 7]
    assert list(split_ptr) == [0, 3, 5, 9]
    assert B._plan_ws(C.byref(st), 128) == st.n_split_items * 128 * 8


@pytest.mark.parametrize("longer", ["split rows", "items"])
def test_agg_plan_fill_with_another_rowptr_fails_inside_its_arrays(longer):
    """A plan filled from a rowptr other than the one it was sized for is rejected, and nothing is
    written past the arrays of the sizes the plan gives (guard words after each stay intact)."""
    lens = np.array([3, 700, 1, 2, 600, 4], np.int32)
    ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    st = B.AggPlanStruct()
    B._check(B._plan_size(ptr.size - 1, ptr.ctypes.data, 512, 256, 0, C.byref(st)), "size")
    more = lens.copy()
    if longer == "split rows":
        more[0] = 900                   # a third split row
    else:
        more[:] = [3, 2500, 0, 2, 0, 4]  # 10 items against 7, one split row against 2
    other = np.concatenate([[0], np.cumsum(more)]).astype(np.int32)
    guard = -7
    items = np.full(4 * st.n_items + 8, guard, np.int32)
    split_row = np.full(st.n_split_rows + 8, guard, np.int32)
    sp = np.full(st.n_split_rows + 1 + 8, guard, np.int32)
    rc = B._plan_fill(other.ctypes.data, C.byref(st), items.ctypes.data, split_row.ctypes.data, sp.ctypes.data)
    assert rc == B.QHA_ERR_INVALID_ARG
    assert (items[4 * st.n_items:] == guard).all()
    assert (split_row[st.n_split_rows:] == guard).all()
    assert (sp[st.n_split_rows + 1:] == guard).all()
    # the rowptr the plan was sized for still fills it
    assert B._plan_fill(ptr.ctypes.data, C.byref(st), items.ctypes.data, split_row.ctypes.data,
                        sp.ctypes.data) == B.QHA_OK


def test_device_calls_reject_bad_arguments_before_any_hip_call():
    q = B._quantize_pack
    # unsupported width
    assert q(FAKE, 24, None, 10, 24, FAKE, FAKE, None, 1, 0, 0, 0, FAKE, FAKE, None) == B.QHA_ERR_UNSUPPORTED
    # leading dimension below d
    assert q(FAKE, 64, None, 10, 128, FAKE, FAKE, None, 1, 0, 0, 0, FAKE, FAKE, None) == B.QHA_ERR_INVALID_ARG
    # misaligned rows
    assert q(FAKE + 4, 128, None, 10, 128, FAKE, FAKE, None, 1, 0, 0, 0, FAKE, FAKE, None) == B.QHA_ERR_INVALID_ARG
    # null outputs, misaligned metadata pairs, neither classes nor a per-row table
    assert q(FAKE, 128, None, 10, 128, FAKE, FAKE, None, 1, 0, 0, 0, None, FAKE, None) == B.QHA_ERR_INVALID_ARG
    assert q(FAKE, 128, None, 10, 128, FAKE, FAKE, None, 1, 0, 0, 0, FAKE, FAKE + 4, None) == B.QHA_ERR_INVALID_ARG
    assert q(FAKE, 128, None, 10, 128, None, None, None, 1, 0, 0, 0, FAKE, FAKE, None) == B.QHA_ERR_INVALID_ARG
    # classes that do not cover the rows, or do not follow each other
    cl = B.pack_classes(np.array([4] * 9, np.uint8), 128)
    assert q(FAKE, 128, None, 10, 128, None, None, C.byref(cl), 1, 0, 0, 0, FAKE, FAKE, None) == B.QHA_ERR_INVALID_ARG
    cl = B.pack_classes(np.array([4] * 5 + [8] * 5, np.uint8), 128)
    cl.base[1] += 1
    assert q(FAKE, 128, None, 10, 128, None, None, C.byref(cl), 1, 0, 0, 0, FAKE, FAKE, None) == B.QHA_ERR_INVALID_ARG
    # node ids overflow 32 bits
    assert q(FAKE, 128, None, 10, 128, FAKE, FAKE, None, 1, 0, 0, 0xFFFFFFFF, FAKE, FAKE, None) == B.QHA_ERR_INVALID_ARG
    # nothing to do is OK without touching the device
    assert q(None, 0, None, 0, 128, None, None, None, 1, 0, 0, 0, None, None, None) == B.QHA_OK

    f = B._dequant_aggregate_fwd
    args = dict(n_rows=10, rowptr=FAKE, colidx=FAKE, w=None, row_ids=None, plan=None, x=FAKE, ldx=128,
                n_inner=5, codes=FAKE, wo=FAKE, bits=FAKE, classes=None, meta=FAKE, n_halo=5, d=128, beta=0, out=FAKE,
                ldo=128, ws=None, wsb=0, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())
    assert call(beta=2) == B.QHA_ERR_INVALID_ARG
    assert call(d=100) == B.QHA_ERR_UNSUPPORTED
    assert call(ldo=130) == B.QHA_ERR_INVALID_ARG
    assert call(codes=None) == B.QHA_ERR_INVALID_ARG
    assert call(meta=FAKE + 4) == B.QHA_ERR_INVALID_ARG
    assert call(rowptr=None) == B.QHA_ERR_INVALID_ARG
    assert call(n_inner=-1) == B.QHA_ERR_INVALID_ARG
    # a plan that skips empty rows cannot be combined with beta = 0
    lens = np.array([0, 600, 3], np.int32)
    ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    st, *_ = _plan_host(ptr, 512, True)
    st.items = st.split_row = st.split_ptr = FAKE
    assert call(n_rows=3, plan=C.byref(st)) == B.QHA_ERR_INVALID_ARG
    st2, *_ = _plan_host(ptr, 512, False)
    st2.items = st2.split_row = st2.split_ptr = FAKE
    # split rows need a workspace
    assert call(n_rows=3, plan=C.byref(st2)) == B.QHA_ERR_WORKSPACE
    # plan built for another row count
    assert call(n_rows=4, plan=C.byref(st2)) == B.QHA_ERR_INVALID_ARG

    g = B._aggregate_bwd
    assert g(10, FAKE, FAKE, None, None, FAKE, 128, 10, 128, 3, FAKE, 128, None, 0, None) == B.QHA_ERR_INVALID_ARG
    assert g(10, FAKE, FAKE, None, None, FAKE, 96, 10, 128, 0, FAKE, 128, None, 0, None) == B.QHA_ERR_INVALID_ARG
    assert B._edge_weights(10, None, FAKE, None, None, FAKE, None) == B.QHA_ERR_INVALID_ARG

    p = B._dense_project
    # contiguous extent of A not a multiple of 4
    assert p(0, 1, 100, 128, 126, FAKE, 128, FAKE, 128, 0, FAKE, 128, 0, None, 0, 1, None, 0, None) == B.QHA_ERR_INVALID_ARG
    # mask prologue without aux
    assert p(0, 0, 100, 128, 128, FAKE, 128, FAKE, 128, 0, FAKE, 128, 1, None, 0, 0, None, 0, None) == B.QHA_ERR_INVALID_ARG
    # split-k reduction without workspace
    assert B.dense_project_workspace(1, 0, 128, 128, 300000) > 0
    assert p(1, 0, 128, 128, 300000, FAKE, 128, FAKE, 128, 0, FAKE, 128, 0, None, 0, 0, None, 0, None) == B.QHA_ERR_WORKSPACE
    assert B._last_error().decode().startswith("workspace")
    assert B._degree_norm(FAKE, 10, 7, FAKE, None) == B.QHA_ERR_INVALID_ARG

    b = B._dense_bwd
    bargs = dict(m=1000, n=128, k=128, dh=FAKE, ldg=128, h=FAKE, ldh=128, a=FAKE, lda=128, w=FAKE, ldw=128,
                 da=FAKE, ldda=128, dw=FAKE, lddw=128, ws=None, wsb=0, s=None)

    def bcall(**kw):
        a = dict(bargs, **kw)
        return b(*a.values())
    # the width-128 panel path needs one float dW partial per block
    assert B.dense_backward_workspace(1000, 128, 128) == 16 * 128 * 128 * 4
    assert B.dense_backward_workspace(300000, 128, 128) == 256 * 128 * 128 * 4
    assert bcall() == B.QHA_ERR_WORKSPACE
    assert bcall(ws=FAKE + 8, wsb=1 << 30) == B.QHA_ERR_INVALID_ARG     # misaligned workspace
    assert bcall(n=126, ldg=126, ldh=126) == B.QHA_ERR_INVALID_ARG     # widths not multiples of 4
    assert bcall(h=FAKE + 4) == B.QHA_ERR_INVALID_ARG                   # misaligned H
    assert bcall(lda=64) == B.QHA_ERR_INVALID_ARG                       # leading dimension below k
    assert bcall(w=None) == B.QHA_ERR_INVALID_ARG
    assert bcall(m=-1) == B.QHA_ERR_INVALID_ARG
    # other widths take the general products, whose dW reduction may split
    assert B.dense_backward_workspace(300000, 256, 512) == B.dense_project_workspace(1, 0, 256, 512, 300000)
    assert bcall(n=256, k=512, ldg=256, ldh=256, lda=512, ldw=512, ldda=512, lddw=512, m=300000) == B.QHA_ERR_WORKSPACE
    assert bcall(n=0) == B.QHA_OK


def test_noalloc_aggregation_rejects_before_any_hip_call():
    """The allocation-free aggregation refuses a plan whose split-row partials exceed its scratch, and
    bad arguments, before it looks anything up on the device."""
    f = B._dequant_aggregate_fwd_noalloc
    lens = np.full(100, 8000, np.int32)                    # 100 rows split into 500 chunks of 16 each
    ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    st, *_ = _plan_host(ptr, 16, False)
    st.items = st.split_row = st.split_ptr = FAKE
    assert B._plan_ws(C.byref(st), 512) > B.NOALLOC_SCRATCH_BYTES
    args = dict(n_rows=100, rowptr=FAKE, colidx=FAKE, w=None, row_ids=None, plan=C.byref(st), x=FAKE, ldx=512,
                n_inner=5, codes=None, wo=None, bits=None, classes=None, meta=None, n_halo=0, d=512, beta=0, out=FAKE,
                ldo=512, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())
    assert call() == B.QHA_ERR_WORKSPACE
    assert "static scratch" in B._last_error().decode()
    assert B._plan_ws(C.byref(st), 128) <= B.NOALLOC_SCRATCH_BYTES
    assert call(d=128, ldx=128, ldo=128, beta=2) == B.QHA_ERR_INVALID_ARG
    assert call(d=128, ldx=128, ldo=96) == B.QHA_ERR_INVALID_ARG
    assert call(d=100) == B.QHA_ERR_UNSUPPORTED
    assert call(n_rows=0) == B.QHA_OK


def test_received_messages_rejected_before_any_hip_call():
    """The received messages of the one-launch transposed gather are checked on the host: null lists,
    a buffer that is the call's own output, misaligned arrays, classes that do not cover the rows."""
    f = B._aggregate_bwd_quantize
    out_codes, out_meta = FAKE, FAKE + 4096
    rs = B.ReceivedStruct(FAKE, FAKE, 5, FAKE + 8192, FAKE + 12288, FAKE, FAKE, None)
    args = dict(n_rows=10, colptr=FAKE, rowidx=FAKE, w=None, plan=None, g=FAKE, ldg=128, n_grad=10, d=128,
                n_stored=5, beta=0, gi=FAKE, ldi=128, bits=FAKE, wo=FAKE, classes=None, seed=1, epoch=0, sid=0,
                base=0, codes=out_codes, meta=out_meta, rcv=C.byref(rs), ws=None, wsb=0, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())

    def with_rs(**fields):
        r = B.ReceivedStruct(*[fields.get(n, getattr(rs, n)) for n, _ in B.ReceivedStruct._fields_])
        return call(rcv=C.byref(r))
    assert with_rs(copy_ptr=None) == B.QHA_ERR_INVALID_ARG
    assert with_rs(copy_idx=None) == B.QHA_ERR_INVALID_ARG
    assert with_rs(codes=None) == B.QHA_ERR_INVALID_ARG
    assert with_rs(n_rows=-1) == B.QHA_ERR_INVALID_ARG
    assert with_rs(codes=out_codes) == B.QHA_ERR_INVALID_ARG
    assert "writes" in B._last_error().decode()
    assert with_rs(meta=out_meta) == B.QHA_ERR_INVALID_ARG
    assert with_rs(meta=FAKE + 12292) == B.QHA_ERR_INVALID_ARG          # (min, scale) pairs misaligned
    assert with_rs(bits=None) == B.QHA_ERR_INVALID_ARG                  # no widths at all
    cl = B.pack_classes(np.array([4] * 4, np.uint8), 128)               # classes of 4 rows, buffer of 5
    assert with_rs(bits=None, word_offset=None, classes=C.pointer(cl)) == B.QHA_ERR_INVALID_ARG
