"""Fused dequantise + aggregate (forward), transposed aggregate (backward) and the received-gradient add
on the GPU against the oracle, on the same seeded inputs (messages quantised by the oracle)."""
import numpy as np
import pytest

import gpu_helpers as H
from oracle import aggregate as OA
from quantized_halo_aggregation_amd import synth

pytestmark = pytest.mark.gpu

SEED = synth.QUANT_SEED

# (n_in, n_h, nnz, d, bits recipe, model, chunk): several tiles, ragged sizes, heavy rows split
CASES = [
    (301, 97, 3000, 16, ("uniform", (1, 2, 4, 8, 32)), "gcn", 512),
    (517, 713, 20000, 32, ("uniform", (1, 2, 4, 8)), "gcn", 32),
    (777, 300, 12000, 64, ("uniform", (1, 2, 4, 8, 32)), "gcn", 64),
    (1003, 301, 30000, 128, ("top", 4, 8, 0.10), "gcn", 64),
    (1003, 301, 30000, 128, ("uniform", (1, 2, 4, 8, 32)), "gcn", 512),
    (401, 203, 8000, 256, ("top", 2, 4, 0.20), "gcn", 100),
    (203, 101, 2000, 512, ("uniform", (1, 2, 4, 8, 32)), "gcn", 16),
    (999, 333, 9000, 128, ("const", 1), "sage", 48),
    (513, 257, 5000, 256, ("const", 1), "sage", 512),
]


def _case_id(c):
    return f"{c[5]}-n{c[0]}-h{c[1]}-d{c[3]}-c{c[6]}"


def _setup(case):
    from quantized_halo_aggregation_amd.pipeline import GpuPartition
    n_in, n_h, nnz, d, bits, model, chunk = case
    wl = synth.small_workload(n_in, n_h, nnz, d, bits=bits, model=model, index=100 + CASES.index(case))
    part = synth.make_partition(wl)
    gp = GpuPartition(part, chunk=chunk)
    return part, gp


@pytest.mark.parametrize("case", CASES, ids=_case_id)
@pytest.mark.parametrize("grouped", [True, False], ids=["width-classes", "offset-table"])
def test_forward_aggregation(case, grouped):
    H.require_gpu()
    import torch
    part, gp = _setup(case)
    gp.set_bits(part.bits, grouped=grouped)
    n_in, d = part.n_in, part.d
    msg = H.oracle_messages(part.x[part.mirror], part.bits, SEED, 0, 0, n_in)
    x_cols = np.concatenate([part.x, msg["received"]])
    if part.wl.model == "gcn":
        ref = OA.gcn_aggregate(part.nbr_ptr, part.nbr_idx, part.deg, x_cols)
        H.note(f"aggregate_fwd {_case_id(case)}")
        out = torch.full((n_in, d), np.nan, dtype=torch.float32, device="cuda")
        gp.aggregate_fwd(H.dev(part.x), H.upload_messages(gp, msg), out)
        H.assert_close(H.host(out), ref, what="aggregate_fwd")
    else:
        ref = OA.mean_aggregate(part.nbr_ptr, part.nbr_idx, x_cols)
        H.note(f"aggregate_fwd sage {_case_id(case)}")
        acat = torch.full((n_in, 2 * d), np.nan, dtype=torch.float32, device="cuda")
        acat[:, :d] = H.dev(part.x)
        gp.aggregate_fwd(acat[:, :d], H.upload_messages(gp, msg), acat[:, d:])
        got = H.host(acat)
        H.assert_close(got[:, d:], ref, what="mean aggregate (strided output)")
        H.assert_bits_equal(got[:, :d], part.x, "self half untouched")


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_backward_aggregation_and_received_add(case):
    H.require_gpu()
    import torch
    part, gp = _setup(case)
    n_in, n_h, d = part.n_in, part.n_h, part.d
    rng = np.random.default_rng(5)
    g = rng.standard_normal((n_in, d)).astype(np.float32)
    if part.wl.model == "gcn":
        ref = OA.gcn_aggregate_t(part.nbr_ptr, part.nbr_idx, part.deg, g)
    else:
        ref = OA.mean_aggregate_t(part.nbr_ptr, part.nbr_idx, g, n_in + n_h)
    H.note(f"aggregate_bwd {_case_id(case)}")
    g_dev = H.dev(g)
    dxh = torch.full((n_h, d), np.nan, dtype=torch.float32, device="cuda")
    gp.aggregate_bwd_halo(g_dev, dxh)
    H.assert_close(H.host(dxh), ref[n_in:], what="aggregate_bwd halo")
    base = rng.standard_normal((n_in, d)).astype(np.float32)
    dxi = H.dev(base)
    gp.aggregate_bwd_inner(g_dev, dxi, 1)
    H.assert_close(H.host(dxi), ref[:n_in] + base.astype(np.float64), what="aggregate_bwd inner (beta=1)")
    dxi0 = torch.full((n_in, d), np.nan, dtype=torch.float32, device="cuda")
    gp.aggregate_bwd_inner(g_dev, dxi0, 0)
    H.assert_close(H.host(dxi0), ref[:n_in], what="aggregate_bwd inner (beta=0)")

    # received halo gradients: quantised by the oracle, dequantised and added on the GPU to the
    # oracle's inner gradients
    halo_grad = ref[n_in:].astype(np.float32)
    msg = H.oracle_messages(halo_grad, part.bits, SEED, 0, 1, n_in)
    start = ref[:n_in].astype(np.float32)
    want = OA.add_received(start, part.mirror, msg["received"])
    dxr = H.dev(start)
    gp.add_received(H.upload_messages(gp, msg), dxr)
    got = H.host(dxr)
    H.assert_close(got, want, what="received add")
    untouched = np.setdiff1d(np.arange(n_in), part.mirror)
    H.assert_bits_equal(got[untouched], start[untouched], "rows without a halo copy")

    # the folded call: the inner columns' gradients and the received messages in one gather
    # (beta = 1 adds both to what the rows hold)
    H.note(f"aggregate_bwd_inner_received {_case_id(case)}")
    omsg = H.upload_messages(gp, msg)
    folded = H.dev(base)
    gp.aggregate_bwd_inner_received(g_dev, omsg, folded, 1)
    H.assert_close(H.host(folded), OA.add_received(ref[:n_in] + base.astype(np.float64), part.mirror,
                                                   msg["received"]), what="folded inner + received (beta=1)")
    folded0 = torch.full((n_in, d), np.nan, dtype=torch.float32, device="cuda")
    gp.aggregate_bwd_inner_received(g_dev, omsg, folded0, 0)
    H.assert_close(H.host(folded0), OA.add_received(ref[:n_in], part.mirror, msg["received"]),
                   what="folded inner + received (beta=0)")


@pytest.mark.parametrize("case", CASES, ids=_case_id)
@pytest.mark.parametrize("grouped", [True, False], ids=["width-classes", "offset-table"])
def test_fused_halo_gradient_quantisation(case, grouped):
    """qha_aggregate_bwd_quantize codes each halo column's gradient exactly as qha_aggregate_bwd
    followed by qha_quantize_pack does (every word and (min, scale) pair, heavy columns split into
    chunks included), and the dequantised codes lie within one quantisation step of the oracle's
    float64 gradients."""
    H.require_gpu()
    import torch
    from oracle import quantize as OQ
    part, gp = _setup(case)
    gp.set_bits(part.bits, grouped=grouped)
    n_in, n_h, d = part.n_in, part.n_h, part.d
    g = np.random.default_rng(9).standard_normal((n_in, d)).astype(np.float32)
    g_dev = H.dev(g)
    H.note(f"aggregate_bwd_quantize {_case_id(case)} grouped={grouped}")
    dxh = torch.empty((n_h, d), dtype=torch.float32, device="cuda")
    gp.aggregate_bwd_halo(g_dev, dxh)
    two = gp.new_messages()
    gp.quantize_send(dxh, None, two, 3, 5)
    fused = gp.new_messages()
    fused.codes.fill_(-559038737)                       # 0xDEADBEEF: every word must be written
    fused.meta.fill_(float("nan"))
    gp.aggregate_bwd_halo_quantize(g_dev, fused, 3, 5)
    words = H.host(fused.codes).view(np.uint32)
    H.assert_bits_equal(words[:gp.total_words], H.host(two.codes).view(np.uint32)[:gp.total_words], "codes")
    H.assert_bits_equal(H.host(fused.meta), H.host(two.meta), "(min, scale)")

    if part.wl.model == "gcn":
        ref = OA.gcn_aggregate_t(part.nbr_ptr, part.nbr_idx, part.deg, g)[n_in:]
    else:
        ref = OA.mean_aggregate_t(part.nbr_ptr, part.nbr_idx, g, n_in + n_h)[n_in:]
    meta = H.host(fused.meta)
    zp, sc = meta[:, 0].astype(np.float64), meta[:, 1].astype(np.float64)
    codes = OQ.unpack(words[:gp.total_words], gp.h_word_offset, part.bits, d)
    deq = OQ.dequantize(codes, meta[:, 1], meta[:, 0], part.bits).astype(np.float64)
    tol = 1e-6 + 1e-5 * np.abs(ref)
    step = sc[:, None] * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - ref) <= step + tol + np.spacing(np.abs(ref).astype(np.float32))), "dequantised codes"
    q = part.bits != 32
    rmin, rmax = ref.min(axis=1), ref.max(axis=1)
    assert np.all(np.abs(zp[q] - rmin[q]) <= 1e-6 + 1e-5 * np.abs(rmin[q])), "zero-points"
    levels = (2.0 ** part.bits[q].astype(np.float64)) - 1
    range_tol = 2e-6 + 2e-5 * np.abs(ref[q]).max(axis=1)          # both ends within the tolerance
    assert np.all(np.abs(sc[q] - (rmax[q] - rmin[q]) / levels) <= range_tol / levels + 3e-7 * sc[q]), "scales"


@pytest.mark.parametrize("case", CASES, ids=_case_id)
@pytest.mark.parametrize("grouped", [True, False], ids=["width-classes", "offset-table"])
@pytest.mark.parametrize("beta", [0, 1])
def test_one_launch_gradients_and_halo_messages(case, grouped, beta):
    """qha_aggregate_bwd_quantize over every column with n_stored = n_in: the inner columns'
    gradients are stored (added to the old rows when beta = 1) and the halo columns' gradients are
    coded in place, bit for bit as the transposed gather followed by qha_quantize_pack (every word
    and (min, scale) pair; heavy columns split into chunks included)."""
    H.require_gpu()
    import torch
    part, gp = _setup(case)
    gp.set_bits(part.bits, grouped=grouped)
    n_in, n_h, d = part.n_in, part.n_h, part.d
    rng = np.random.default_rng(11)
    g_dev = H.dev(rng.standard_normal((n_in, d)).astype(np.float32))
    old = rng.standard_normal((n_in, d)).astype(np.float32)
    H.note(f"one-launch aggregate_bwd_quantize {_case_id(case)} grouped={grouped} beta={beta}")
    dxc = torch.full((n_in + n_h, d), np.nan, dtype=torch.float32, device="cuda")
    gp.aggregate_bwd_all(g_dev, dxc)
    two = gp.new_messages()
    gp.quantize_send(dxc[n_in:], None, two, 4, 7)
    ref_in = H.dev(old)
    gp.aggregate_bwd_inner(g_dev, ref_in, 1)
    fused = gp.new_messages()
    fused.codes.fill_(-559038737)                       # 0xDEADBEEF: every word must be written
    fused.meta.fill_(float("nan"))
    dxi = H.dev(old) if beta else torch.full((n_in, d), np.nan, dtype=torch.float32, device="cuda")
    gp.aggregate_bwd_all_quantize(g_dev, dxi, fused, 4, 7, beta)
    want = H.host(ref_in) if beta else H.host(dxc)[:n_in]
    H.assert_bits_equal(H.host(dxi), want, "inner gradients")
    H.assert_bits_equal(H.host(fused.codes).view(np.uint32)[:gp.total_words],
                        H.host(two.codes).view(np.uint32)[:gp.total_words], "codes")
    H.assert_bits_equal(H.host(fused.meta), H.host(two.meta), "(min, scale)")


# widths of an earlier epoch's messages: each class moved to another width, so that the received
# buffer's layout differs from the one the call writes
_EARLIER = {1: 2, 2: 4, 4: 8, 8: 32, 32: 1}


@pytest.mark.parametrize("case", CASES, ids=_case_id)
@pytest.mark.parametrize("layouts", [(True, True), (False, True), (True, False)],
                         ids=["classes", "offset-table-out", "offset-table-received"])
@pytest.mark.parametrize("beta", [0, 1])
def test_one_launch_adds_received_messages(case, layouts, beta):
    """qha_aggregate_bwd_quantize with messages received earlier (at other widths, in their own
    layout): every inner row equals, bit for bit, the launch without them followed by the received
    add (qha_dequant_aggregate_fwd over the copy lists); the messages it codes are unchanged; and
    the inner rows match the oracle's transposed aggregate plus its received add.  n_h > n_in cases
    give inner nodes several copies; heavy columns split into chunks go through the combine."""
    H.require_gpu()
    import torch
    part, gp = _setup(case)
    grouped_out, grouped_rcv = layouts
    n_in, n_h, d = part.n_in, part.n_h, part.d
    rng = np.random.default_rng(13)
    g = rng.standard_normal((n_in, d)).astype(np.float32)
    old = rng.standard_normal((n_in, d)).astype(np.float32)
    earlier = np.array([_EARLIER[int(b)] for b in part.bits], np.uint8)
    gp.set_bits(earlier, grouped=grouped_rcv)
    rows = rng.standard_normal((n_h, d)).astype(np.float32)
    msg = H.oracle_messages(rows, earlier, SEED, 2, 9, n_in)
    rcv = H.upload_messages(gp, msg)
    rcv.layout = gp.layout
    gp.set_bits(part.bits, grouped=grouped_out)
    g_dev = H.dev(g)
    H.note(f"one-launch with received messages {_case_id(case)} layouts={layouts} beta={beta}")

    start = lambda: H.dev(old) if beta else torch.full((n_in, d), np.nan, dtype=torch.float32, device="cuda")
    two_in, two_msg = start(), gp.new_messages()
    gp.aggregate_bwd_all_quantize(g_dev, two_in, two_msg, 4, 7, beta)
    gp.add_received(rcv, two_in)
    one_in, one_msg = start(), gp.new_messages()
    one_msg.codes.fill_(-559038737)
    gp.aggregate_bwd_all_quantize(g_dev, one_in, one_msg, 4, 7, beta, received=rcv)
    H.assert_bits_equal(H.host(one_in), H.host(two_in), "inner rows with received messages")
    H.assert_bits_equal(H.host(one_msg.codes).view(np.uint32)[:gp.total_words],
                        H.host(two_msg.codes).view(np.uint32)[:gp.total_words], "codes")
    H.assert_bits_equal(H.host(one_msg.meta), H.host(two_msg.meta), "(min, scale)")

    if part.wl.model == "gcn":
        t = OA.gcn_aggregate_t(part.nbr_ptr, part.nbr_idx, part.deg, g)[:n_in]
    else:
        t = OA.mean_aggregate_t(part.nbr_ptr, part.nbr_idx, g, n_in + n_h)[:n_in]
    stored = (old.astype(np.float64) + t) if beta else t
    H.assert_close(H.host(one_in), OA.add_received(stored, part.mirror, msg["received"]),
                   what="inner rows vs the oracle")


def test_one_launch_over_rows_beyond_4gib_matches_the_rows_kernel():
    """Gradient rows spanning more than 4 GiB (rows 4.4 MB apart) take the general kernel, with 64-bit
    addresses, instead of the plain-row kernel's 32-bit buffer offsets.  The one launch stores the
    inner rows (beta = 0 and 1), codes the halo rows with per-row draws, adds earlier messages to the
    stored rows, and combines the split heavy columns.  Every output equals, bit for bit, the same
    call on compact rows, which takes the plain-row kernel."""
    H.require_gpu()
    import torch
    part, gp = _setup(CASES[3])
    n_in, n_h, d = part.n_in, part.n_h, part.d
    ld = 1_100_000
    assert (n_in - 1) * ld * 4 > 0xFFFFFFFF
    rng = np.random.default_rng(17)
    g = rng.standard_normal((n_in, d)).astype(np.float32)
    old = rng.standard_normal((n_in, d)).astype(np.float32)
    earlier = np.array([_EARLIER[int(b)] for b in part.bits], np.uint8)
    gp.set_bits(earlier)
    rcv = H.upload_messages(gp, H.oracle_messages(rng.standard_normal((n_h, d)).astype(np.float32), earlier, SEED,
                                                  2, 9, n_in))
    rcv.layout = gp.layout
    gp.set_bits(part.bits)
    H.note(f"one launch over gradient rows {ld * 4} bytes apart (general kernel)")
    big = torch.empty((n_in, ld), dtype=torch.float32, device="cuda")
    big[:, :d] = H.dev(g)
    outs = []
    for src in (big[:, :d], H.dev(g)):
        for beta in (0, 1):
            dxi = H.dev(old) if beta else torch.full((n_in, d), np.nan, dtype=torch.float32, device="cuda")
            msg = gp.new_messages()
            gp.aggregate_bwd_all_quantize(src, dxi, msg, 4, 7, beta, received=rcv)
            outs.append((H.host(dxi), H.host(msg.codes).view(np.uint32)[:gp.total_words], H.host(msg.meta)))
    del big
    for beta in (0, 1):
        for what, a, b in zip(("inner rows", "codes", "(min, scale)"), outs[beta], outs[2 + beta]):
            H.assert_bits_equal(a, b, f"{what}, beta = {beta}: rows beyond 4 GiB against compact rows")


def test_deterministic_repeats():
    H.require_gpu()
    import torch
    part, gp = _setup(CASES[3])
    msg = H.upload_messages(gp, H.oracle_messages(part.x[part.mirror], part.bits, SEED, 0, 0, part.n_in))
    x = H.dev(part.x)
    outs = []
    H.note("aggregate determinism")
    for _ in range(3):
        out = torch.empty(part.n_in, part.d, dtype=torch.float32, device="cuda")
        gp.aggregate_fwd(x, msg, out)
        outs.append(H.host(out))
    assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])


def test_plain_rows_and_degenerate_inputs():
    """No plan (one item per row), rows without edges, unsorted widths, empty calls, b = 32 halos,
    explicit edge weights."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng(9)
    d, n_inner, n_halo = 128, 40, 30
    lens = rng.integers(0, 9, size=25)
    lens[[0, 7, 24]] = 0
    ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    idx = np.concatenate([np.sort(rng.choice(n_inner + n_halo, size=l, replace=False)) for l in lens]).astype(np.int32)
    B.validate_csr(ptr, idx, n_inner + n_halo)
    x = rng.standard_normal((n_inner, d)).astype(np.float32)
    hx = rng.standard_normal((n_halo, d)).astype(np.float32)
    bits = rng.choice(np.array([1, 2, 4, 8, 32], np.uint8), size=n_halo)
    msg = H.oracle_messages(hx, bits, 11, 0, 0, n_inner)
    off, _ = B.pack_layout(bits, d)
    r = rng.random(25).astype(np.float32)
    c = rng.random(n_inner + n_halo).astype(np.float32)
    rows = np.repeat(np.arange(25), lens)
    w_ref = (r[rows] * c[idx]).astype(np.float32)            # float32 product, as documented
    H.note("edge weights")
    w = torch.empty(idx.size, dtype=torch.float32, device="cuda")
    B.edge_weights(H.dev(ptr), H.dev(idx), H.dev(r), H.dev(c), w)
    H.assert_bits_equal(H.host(w), w_ref, "edge weights")
    x_cols = np.concatenate([x, msg["received"]]).astype(np.float64)
    ref = np.zeros((25, d))
    np.add.at(ref, rows, w_ref.astype(np.float64)[:, None] * x_cols[idx])
    H.note("aggregate plain rows")
    out = torch.full((25, d), np.nan, dtype=torch.float32, device="cuda")
    B.dequant_aggregate_fwd(H.dev(ptr), H.dev(idx), w, None, H.dev(x), n_inner,
                            H.dev(msg["words"].view(np.int32)), H.dev(off.view(np.int32)), H.dev(bits), None,
                            H.dev(np.stack([msg["zero_point"], msg["scale"]], 1)), n_halo, 0, out)
    got = H.host(out)
    H.assert_close(got, ref, what="plain rows")
    assert not got[[0, 7, 24]].any()
    # zero rows: nothing happens
    B.dequant_aggregate_fwd(H.dev(ptr[:1]), H.dev(idx), None, None, H.dev(x), n_inner, None, None, None, None, None,
                            0, 0, out, n_rows=0)
    # no halo at all: only inner columns, unit weights
    keep = idx < n_inner
    cnt = np.bincount(rows[keep], minlength=25)
    inner_only = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    out2 = torch.full((25, d), np.nan, dtype=torch.float32, device="cuda")
    B.dequant_aggregate_fwd(H.dev(inner_only), H.dev(idx[keep]), None, None, H.dev(x), n_inner, None, None, None, None,
                            None, 0, 0, out2)
    ref2 = np.zeros((25, d))
    np.add.at(ref2, rows[keep], x[idx[keep]].astype(np.float64))
    H.assert_close(H.host(out2), ref2, what="inner-only rows, unit weights")


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256, 512])
@pytest.mark.parametrize("grouped", [True, False], ids=["width-classes", "offset-table"])
@pytest.mark.parametrize("beta", [0, 1])
def test_dequantised_halo_rows_are_exact(d, grouped, beta):
    """A row whose one neighbour is a halo node, at unit weight, is that node's received row: the
    message format's scale * q + min with both roundings in float32 (not one fused multiply-add),
    raw floats at b = 32, bit for bit (beta = 1 adds it to zeros)."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng(31 + d)
    n_h, n_inner = 300, 7
    bits = rng.choice(np.array([1, 2, 4, 8, 32], np.uint8), size=n_h)
    if grouped:
        bits = np.sort(bits)[::-1].copy()
    hx = (rng.standard_normal((n_h, d)) * rng.uniform(0.01, 100.0, size=(n_h, 1))).astype(np.float32)
    msg = H.oracle_messages(hx, bits, 77, 3, 1, n_inner)
    off, _ = B.pack_layout(bits, d)
    classes = B.pack_classes(bits, d) if grouped else None
    assert (classes is not None) == grouped
    ptr = np.arange(n_h + 1, dtype=np.int32)
    idx = (n_inner + rng.permutation(n_h)).astype(np.int32)
    x = rng.standard_normal((n_inner, d)).astype(np.float32)
    meta = np.stack([msg["zero_point"], msg["scale"]], 1).astype(np.float32)
    words = msg["words"] if msg["words"].size else np.zeros(1, np.uint32)
    H.note(f"exact dequantisation d={d} grouped={grouped} beta={beta}")
    out = torch.zeros((n_h, d), dtype=torch.float32, device="cuda") if beta else \
        torch.full((n_h, d), np.nan, dtype=torch.float32, device="cuda")
    B.dequant_aggregate_fwd(H.dev(ptr), H.dev(idx), None, B.AggPlan(ptr), H.dev(x), n_inner,
                            H.dev(words.view(np.int32)), H.dev(off.view(np.int32)), H.dev(bits), classes, H.dev(meta),
                            n_h, beta, out)
    H.assert_bits_equal(H.host(out), msg["received"][idx - n_inner], "dequantised rows")


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256, 512])
@pytest.mark.parametrize("beta", [0, 1])
@pytest.mark.parametrize("weighted, with_ids", [(False, True), (True, True), (False, False)],
                         ids=["ids", "weights-ids", "no-ids"])
def test_one_edge_rows_received_add(d, beta, weighted, with_ids):
    """A gather whose every row holds one halo edge (the received add when each inner node has one
    halo copy) gives old + w * message row rounded once, bit for bit: widths mixed in runs, raw float
    rows, a ragged row count, messages that are not added anywhere, rows of out left alone."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng(900 + d + 7 * beta)
    n_h = 1531                                  # several work items at every d, ragged tail
    n_out = n_h + 211
    bits = np.repeat(np.array([8, 32, 4, 1, 2, 4], np.uint8), [300, 101, 400, 333, 200, 197])
    assert bits.size == n_h
    hx = (rng.standard_normal((n_h, d)) * rng.uniform(0.01, 50.0, size=(n_h, 1))).astype(np.float32)
    msg = H.oracle_messages(hx, bits, 91, 2, 1, 4000)
    classes = B.pack_classes(bits, d)
    n_rows = n_h - 17
    ptr = np.arange(n_rows + 1, dtype=np.int32)
    idx = rng.permutation(n_h)[:n_rows].astype(np.int32)
    ids = rng.permutation(n_out)[:n_rows].astype(np.int32) if with_ids else None
    w = rng.uniform(-2.0, 2.0, size=n_rows).astype(np.float32) if weighted else None
    meta = np.stack([msg["zero_point"], msg["scale"]], 1).astype(np.float32)
    start = rng.standard_normal((n_out, d)).astype(np.float32)
    rows = ids if with_ids else np.arange(n_rows)
    rec = msg["received"][idx].astype(np.float64)
    term = rec * (w.astype(np.float64)[:, None] if weighted else 1.0)
    want = start.copy() if beta else np.full((n_out, d), np.nan, np.float32)
    want[rows] = (start[rows].astype(np.float64) + term if beta else term).astype(np.float32)

    H.note(f"one-edge rows d={d} beta={beta} weighted={weighted} ids={with_ids}")
    out = H.dev(start) if beta else torch.full((n_out, d), np.nan, dtype=torch.float32, device="cuda")
    B.dequant_aggregate_fwd(H.dev(ptr), H.dev(idx), None if w is None else H.dev(w), B.AggPlan(ptr), None, 0,
                            H.dev(msg["words"].view(np.int32)), None, None, classes, H.dev(meta), n_h, beta, out,
                            row_ids=None if ids is None else H.dev(ids))
    H.assert_bits_equal(H.host(out), want, "one-edge rows against old + w * message")


def test_plain_gather_beyond_32bit_offsets():
    """Rows of x more than 4 GiB apart (a row pitch of 2^24 floats): the gather takes its 64-bit
    addressing path and still sums the right rows."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    d, n_x, pitch = 128, 65, 1 << 24
    rng = np.random.default_rng(12)
    big = torch.empty(n_x * pitch, dtype=torch.float32, device="cuda")
    xv = rng.standard_normal((n_x, d)).astype(np.float32)
    xs = big.view(n_x, pitch)[:, :d]
    xs.copy_(H.dev(xv))
    lens = rng.integers(1, 12, size=40)
    ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    idx = rng.integers(0, n_x, size=int(ptr[-1])).astype(np.int32)
    idx[:3] = n_x - 1                                      # the last row, past 4 GiB
    w = rng.random(idx.size).astype(np.float32)
    rows = np.repeat(np.arange(40), lens)
    ref = np.zeros((40, d))
    np.add.at(ref, rows, w.astype(np.float64)[:, None] * xv[idx].astype(np.float64))
    H.note("plain gather, 64-bit offsets")
    out = torch.full((40, d), np.nan, dtype=torch.float32, device="cuda")
    B.dequant_aggregate_fwd(H.dev(ptr), H.dev(idx), H.dev(w), B.AggPlan(ptr), xs, n_x, None, None, None, None, None,
                            0, 0, out)
    H.assert_close(H.host(out), ref, what="gather over a 4.3 GB row pitch")
    ga = torch.full((40, d), np.nan, dtype=torch.float32, device="cuda")
    B.aggregate_bwd(H.dev(ptr), H.dev(idx), H.dev(w), B.AggPlan(ptr), xs, n_x, 0, ga)
    H.assert_close(H.host(ga), ref, what="transposed-call form, same rows")
    del big
    torch.cuda.empty_cache()


def test_grouped_gather_with_buffers_far_apart():
    """Inner rows and the received message more than 4 GiB apart: the grouped gather cannot address
    them from one base and takes its per-buffer path, with the same result as when they are close."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    part, gp = _setup(CASES[3])
    n_in, n_h, d = part.n_in, part.n_h, part.d
    msg = H.oracle_messages(part.x[part.mirror], part.bits, SEED, 0, 0, n_in)
    x_cols = np.concatenate([part.x, msg["received"]])
    ref = OA.gcn_aggregate(part.nbr_ptr, part.nbr_idx, part.deg, x_cols)
    words = msg["words"].view(np.int32)
    meta = np.stack([msg["zero_point"], msg["scale"]], 1).astype(np.float32).reshape(-1)
    gap = (5 << 30) // 4                                    # 5 GiB of float32 between them
    big = torch.empty(gap + words.size + meta.size + 64, dtype=torch.float32, device="cuda")
    xs = big[:n_in * d].view(n_in, d)
    xs.copy_(H.dev(part.x))
    codes = big[gap:gap + words.size].view(torch.int32)
    codes.copy_(H.dev(words))
    mt = big[gap + words.size + 16:gap + words.size + 16 + meta.size]
    mt.copy_(H.dev(meta))
    assert gp.classes is not None
    H.note("grouped gather, buffers 5 GiB apart")
    out = torch.full((n_in, d), np.nan, dtype=torch.float32, device="cuda")
    B.dequant_aggregate_fwd(gp.rowptr, gp.colidx, gp.w_fwd, gp.plan_fwd, xs, n_in, codes, gp.word_offset, gp.bits,
                            gp.classes, mt.view(-1, 2), n_h, 0, out, workspace=gp.agg_ws)
    got = H.host(out)
    H.assert_close(got, ref, what="grouped gather, far buffers")
    near = torch.full((n_in, d), np.nan, dtype=torch.float32, device="cuda")
    gp.aggregate_fwd(H.dev(part.x), H.upload_messages(gp, msg), near)
    H.assert_bits_equal(got, H.host(near), "far and near buffers give the same bits")
    del big, xs, codes, mt
    torch.cuda.empty_cache()
