"""qha_dense_project and qha_dense_backward (float32 products on the matrix cores) against the
oracle's float64 projection and gradients, and their error against float64."""
import numpy as np
import pytest

import gpu_helpers as H
from oracle import dense as OD

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,d_in,d_out", [(1, 16, 16), (1001, 16, 16), (777, 64, 64), (3001, 128, 128),
                                          (1, 128, 128), (65, 128, 128), (70001, 128, 128),
                                          (1000, 256, 256), (513, 512, 256), (130, 32, 48), (300, 64, 512),
                                          (1001, 128, 516)])
def test_forward_projection_relu(m, d_in, d_out):
    """d_in = d_out = 128 runs the row-panel kernel (W's parts on chip; ragged last panel, several
    panels per block at m = 70001); beta = 1 always takes the general kernel, whose outputs of 512
    columns or more use 256-wide block tiles (a ragged last tile at 516)."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng(m + d_in)
    a = rng.standard_normal((m, d_in)).astype(np.float32)
    w = (rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)).astype(np.float32)
    ref = OD.project(a, w)
    H.note(f"dense fwd m={m} {d_in}->{d_out}")
    c = torch.full((m, d_out), np.nan, dtype=torch.float32, device="cuda")
    B.dense_project(0, 1, H.dev(a), H.dev(w), 0, c, epilogue=B.EPI_RELU)
    H.assert_close(H.host(c), ref, what="relu(A W^T)")
    # no epilogue, accumulate into C
    c0 = rng.standard_normal((m, d_out)).astype(np.float32)
    c = H.dev(c0)
    B.dense_project(0, 1, H.dev(a), H.dev(w), 1, c)
    H.assert_close(H.host(c), a.astype(np.float64) @ w.T.astype(np.float64) + c0, what="C + A W^T")


@pytest.mark.parametrize("m,d_in,d_out", [(1001, 16, 16), (3001, 128, 128), (20000, 128, 128),
                                          (4099, 512, 256), (70000, 256, 256), (777, 516, 64)])
def test_backward_projection(m, d_in, d_out):
    """dA = (dH * [H > 0]) W and dW = (dH * [H > 0])^T A; large m exercises the split-k reduction."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng(m * 3 + d_out)
    a = rng.standard_normal((m, d_in)).astype(np.float32)
    w = (rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)).astype(np.float32)
    h = OD.project(a, w).astype(np.float32)
    dh = rng.standard_normal((m, d_out)).astype(np.float32)
    da_ref, dw_ref = OD.project_backward(a, w, h, dh)
    ws_bytes = max(B.dense_project_workspace(0, 0, m, d_in, d_out), B.dense_project_workspace(1, 0, d_out, d_in, m))
    ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device="cuda")
    H.note(f"dense bwd m={m} {d_in}->{d_out} ws={ws_bytes}")
    dh_d, h_d, a_d, w_d = H.dev(dh), H.dev(h), H.dev(a), H.dev(w)
    da = torch.full((m, d_in), np.nan, dtype=torch.float32, device="cuda")
    B.dense_project(0, 0, dh_d, w_d, 0, da, prologue=B.PRO_RELU_MASK, aux=h_d, workspace=ws)
    H.assert_close(H.host(da), da_ref, what="dA")
    dw = torch.full((d_out, d_in), np.nan, dtype=torch.float32, device="cuda")
    B.dense_project(1, 0, dh_d, a_d, 0, dw, prologue=B.PRO_RELU_MASK, aux=h_d, workspace=ws)
    got = H.host(dw)
    H.assert_close_normwise(got, dw_ref, what="dW")
    # deterministic: the split-k partials are summed in a fixed order
    dw2 = torch.empty_like(dw)
    B.dense_project(1, 0, dh_d, a_d, 0, dw2, prologue=B.PRO_RELU_MASK, aux=h_d, workspace=ws)
    assert np.array_equal(H.host(dw2).view(np.uint32), got.view(np.uint32))


def test_strided_operands_and_empty_reduction():
    """Operands that are column slices of wider buffers (the GraphSAGE concat layout), and k = 0."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng(3)
    m, d = 999, 128
    acat = rng.standard_normal((m, 2 * d)).astype(np.float32)
    w = (rng.standard_normal((d, 2 * d)) / 16).astype(np.float32)
    big = torch.full((m, 3 * d), np.nan, dtype=torch.float32, device="cuda")
    out = big[:, d:2 * d]
    H.note("dense strided")
    B.dense_project(0, 1, H.dev(acat), H.dev(w), 0, out, epilogue=B.EPI_RELU)
    got = H.host(big)
    H.assert_close(got[:, d:2 * d], OD.project(acat, w), what="strided C")
    assert np.isnan(got[:, :d]).all() and np.isnan(got[:, 2 * d:]).all()
    a_d = H.dev(acat)
    c = torch.full((m, d), np.nan, dtype=torch.float32, device="cuda")
    B.dense_project(0, 1, a_d[:, :d], H.dev(np.ascontiguousarray(w[:, d:])), 0, c)
    H.assert_close(H.host(c), acat[:, :d].astype(np.float64) @ w[:, d:].T.astype(np.float64), what="strided A")
    # the width-128 row-panel kernel with strided A and C
    big2 = torch.full((m, 3 * d), np.nan, dtype=torch.float32, device="cuda")
    B.dense_project(0, 1, a_d[:, d:], H.dev(np.ascontiguousarray(w[:, :d])), 0, big2[:, d:2 * d], epilogue=B.EPI_RELU)
    got2 = H.host(big2)
    H.assert_close(got2[:, d:2 * d], OD.project(acat[:, d:], np.ascontiguousarray(w[:, :d])), what="panel strided")
    assert np.isnan(got2[:, :d]).all() and np.isnan(got2[:, 2 * d:]).all()
    # an empty reduction writes zeros (then the epilogue)
    z = torch.full((m, d), np.nan, dtype=torch.float32, device="cuda")
    B.dense_project(0, 1, a_d[:, :0], torch.empty((d, 0), dtype=torch.float32, device="cuda"), 0, z)
    assert not H.host(z).any()


@pytest.mark.parametrize("m,d_in,d_out", [(1, 128, 128), (63, 128, 128), (65, 128, 128), (3001, 128, 128),
                                          (70001, 128, 128), (1001, 16, 16), (2000, 256, 256), (4099, 512, 256),
                                          (5000, 256, 128), (3000, 512, 512), (140001, 512, 256), (5, 256, 256)])
def test_fused_dense_backward(m, d_in, d_out):
    """qha_dense_backward: dA and dW in one call.  Width 128 runs the fused row-panel kernel (ragged
    panels, several panels per block at m = 70001, strided dH / H rows); other widths the general
    products, with dW by row panels where d_out is a multiple of 128 and d_in of 256 (at m = 140001
    with more row ranges than blocks fill the chip, at m = 5 with ranges that hold no rows).
    Bitwise repeatable."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng(m * 7 + d_in)
    a = rng.standard_normal((m, d_in)).astype(np.float32)
    w = (rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)).astype(np.float32)
    h = OD.project(a, w).astype(np.float32)
    dh = rng.standard_normal((m, d_out)).astype(np.float32)
    da_ref, dw_ref = OD.project_backward(a, w, h, dh)
    ws_bytes = B.dense_backward_workspace(m, d_out, d_in)
    ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device="cuda")
    H.note(f"dense_backward m={m} {d_in}->{d_out} ws={ws_bytes}")
    # dH and H as column slices of wider buffers (row stride 2 * d_out)
    wide = torch.full((m, 4 * d_out), np.nan, dtype=torch.float32, device="cuda")
    wide[:, :d_out] = H.dev(dh)
    wide[:, 2 * d_out:3 * d_out] = H.dev(h)
    dh_d, h_d = wide[:, :d_out], wide[:, 2 * d_out:3 * d_out]
    a_d, w_d = H.dev(a), H.dev(w)
    da = torch.full((m, d_in), np.nan, dtype=torch.float32, device="cuda")
    dw = torch.full((d_out, d_in), np.nan, dtype=torch.float32, device="cuda")
    B.dense_backward(dh_d, h_d, a_d, w_d, da, dw, workspace=ws)
    got_da, got_dw = H.host(da), H.host(dw)
    H.assert_close(got_da, da_ref, what="dA")
    H.assert_close_normwise(got_dw, dw_ref, what="dW")
    da2, dw2 = torch.empty_like(da), torch.empty_like(dw)
    B.dense_backward(dh_d, h_d, a_d, w_d, da2, dw2, workspace=ws)
    assert np.array_equal(H.host(da2).view(np.uint32), got_da.view(np.uint32))
    assert np.array_equal(H.host(dw2).view(np.uint32), got_dw.view(np.uint32))


def test_dense_backward_of_no_rows_writes_zero_weight_gradient():
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    e = torch.empty((0, 128), dtype=torch.float32, device="cuda")
    w = torch.ones((128, 128), dtype=torch.float32, device="cuda")
    dw = torch.full((128, 128), np.nan, dtype=torch.float32, device="cuda")
    H.note("dense_backward m=0")
    B.dense_backward(e, e, e, w, e, dw)
    assert not H.host(dw).any()


@pytest.mark.parametrize("dist", ["normal", "wide-range", "cancelling"])
def test_forward_error_is_float32_class(dist):
    """The width-128 forward's error against float64, relative to sum_k |a_k w_k| per element, stays
    within 8 units of float32 rounding (2^-24) on well-scaled, wide-range (e^+-8 per element) and
    cancelling rows: the products are formed at float32 accuracy whatever units compute them."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng({"normal": 1, "wide-range": 2, "cancelling": 3}[dist])
    m, d = 3001, 128
    if dist == "normal":
        a = rng.standard_normal((m, d))
    elif dist == "wide-range":
        a = rng.standard_normal((m, d)) * np.exp(rng.uniform(-8, 8, (m, d)))
    else:
        a = np.repeat(rng.standard_normal((m, 1)), d, 1) * np.where(np.arange(d) % 2, 1, -1) + \
            1e-3 * rng.standard_normal((m, d))
    a = a.astype(np.float32)
    w = (rng.standard_normal((d, d)) / 11.3).astype(np.float32)
    H.note(f"forward error bound, {dist}")
    h = torch.full((m, d), np.nan, dtype=torch.float32, device="cuda")
    B.dense_project(0, 1, H.dev(a), H.dev(w), 0, h)
    got = H.host(h).astype(np.float64)
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    scale = np.abs(a.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    err = np.abs(got - ref) / scale
    assert err.max() <= 8 * 2.0 ** -24, f"max error {err.max() * 2**24:.2f} units of 2^-24"


@pytest.mark.parametrize("dist", ["normal", "wide-range", "cancelling"])
def test_backward_error_is_float32_class(dist):
    """The width-128 backward's error against float64, relative to the sum of |terms| per element:
    dA within 8 units of 2^-24 (chains of 32 products folded into float64, as in the forward), dW
    within 16 units (float32 sums over each block's rows, at most 64 rows per block at m = 3001,
    then float64 across blocks; measured at most 2.7)."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng({"normal": 11, "wide-range": 12, "cancelling": 13}[dist])
    m, d = 3001, 128
    if dist == "normal":
        a = rng.standard_normal((m, d))
        dh = rng.standard_normal((m, d))
    elif dist == "wide-range":
        a = rng.standard_normal((m, d)) * np.exp(rng.uniform(-8, 8, (m, d)))
        dh = rng.standard_normal((m, d)) * np.exp(rng.uniform(-8, 8, (m, d)))
    else:
        a = np.repeat(rng.standard_normal((m, 1)), d, 1) * np.where(np.arange(d) % 2, 1, -1) + \
            1e-3 * rng.standard_normal((m, d))
        dh = np.repeat(rng.standard_normal((1, d)), m, 0) * np.where(np.arange(m) % 2, 1, -1)[:, None] + \
            1e-3 * rng.standard_normal((m, d))
    a = a.astype(np.float32)
    dh = dh.astype(np.float32)
    w = (rng.standard_normal((d, d)) / 11.3).astype(np.float32)
    h = np.where(rng.random((m, d)) < 0.5, 0.0, 1.0).astype(np.float32)     # the ReLU mask's pattern
    H.note(f"backward error bound, {dist}")
    ws = torch.empty(B.dense_backward_workspace(m, d, d) // 4 + 1, dtype=torch.float32, device="cuda")
    da = torch.full((m, d), np.nan, dtype=torch.float32, device="cuda")
    dw = torch.full((d, d), np.nan, dtype=torch.float32, device="cuda")
    B.dense_backward(H.dev(dh), H.dev(h), H.dev(a), H.dev(w), da, dw, workspace=ws)
    z = np.where(h > 0, dh, 0.0).astype(np.float64)
    ref_da, sc_da = z @ w.astype(np.float64), np.abs(z) @ np.abs(w.astype(np.float64))
    ref_dw, sc_dw = z.T @ a.astype(np.float64), np.abs(z).T @ np.abs(a.astype(np.float64))
    e_da = np.abs(H.host(da).astype(np.float64) - ref_da) / np.maximum(sc_da, 1e-300)
    e_dw = np.abs(H.host(dw).astype(np.float64) - ref_dw) / np.maximum(sc_dw, 1e-300)
    H.note(f"  dA max {e_da.max() * 2**24:.2f}, dW max {e_dw.max() * 2**24:.2f} units of 2^-24")
    assert e_da.max() <= 8 * 2.0 ** -24, f"dA: max error {e_da.max() * 2**24:.2f} units of 2^-24"
    assert e_dw.max() <= 16 * 2.0 ** -24, f"dW: max error {e_dw.max() * 2**24:.2f} units of 2^-24"


@pytest.mark.parametrize("m,d_in,d_out", [(3001, 256, 256), (2000, 512, 256), (1001, 16, 16), (140001, 512, 256)])
def test_general_width_error_is_float32_class(m, d_in, d_out):
    """The tiled products at widths other than 128 (split parts on the bf16 matrix cores, 32-k
    chains folded into float64): the forward and dA within 8 units of 2^-24 of the sum of |terms|
    per element, dW within 16 units, on wide-range operands (e^+-8 per element)."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng(m + d_in)
    a = (rng.standard_normal((m, d_in)) * np.exp(rng.uniform(-8, 8, (m, d_in)))).astype(np.float32)
    w = (rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)).astype(np.float32)
    dh = (rng.standard_normal((m, d_out)) * np.exp(rng.uniform(-8, 8, (m, d_out)))).astype(np.float32)
    h = np.where(rng.random((m, d_out)) < 0.5, 0.0, 1.0).astype(np.float32)
    H.note(f"general-width error bound m={m} {d_in}->{d_out}")
    out = torch.full((m, d_out), np.nan, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(B.dense_project_workspace(0, 1, m, d_out, d_in), 4) // 4, dtype=torch.float32, device="cuda")
    B.dense_project(0, 1, H.dev(a), H.dev(w), 0, out, workspace=ws)
    a64, w64 = a.astype(np.float64), w.astype(np.float64)
    e_f = np.abs(H.host(out).astype(np.float64) - a64 @ w64.T) / np.maximum(np.abs(a64) @ np.abs(w64).T, 1e-300)
    wsb = torch.empty(B.dense_backward_workspace(m, d_out, d_in) // 4 + 1, dtype=torch.float32, device="cuda")
    da = torch.full((m, d_in), np.nan, dtype=torch.float32, device="cuda")
    dw = torch.full((d_out, d_in), np.nan, dtype=torch.float32, device="cuda")
    B.dense_backward(H.dev(dh), H.dev(h), H.dev(a), H.dev(w), da, dw, workspace=wsb)
    z = np.where(h > 0, dh, 0.0).astype(np.float64)
    e_da = np.abs(H.host(da).astype(np.float64) - z @ w64) / np.maximum(np.abs(z) @ np.abs(w64), 1e-300)
    e_dw = np.abs(H.host(dw).astype(np.float64) - z.T @ a64) / np.maximum(np.abs(z).T @ np.abs(a64), 1e-300)
    H.note(f"  forward {e_f.max() * 2**24:.2f}, dA {e_da.max() * 2**24:.2f}, dW {e_dw.max() * 2**24:.2f} units")
    assert e_f.max() <= 8 * 2.0 ** -24, f"forward: {e_f.max() * 2**24:.2f} units of 2^-24"
    assert e_da.max() <= 8 * 2.0 ** -24, f"dA: {e_da.max() * 2**24:.2f} units of 2^-24"
    assert e_dw.max() <= 16 * 2.0 ** -24, f"dW: {e_dw.max() * 2**24:.2f} units of 2^-24"


@pytest.mark.parametrize("m,n,k,tb,mask,beta", [(20000, 256, 512, 1, False, 0), (20000, 512, 256, 0, True, 0),
                                                (16384, 516, 64, 1, False, 0), (17001, 52, 132, 0, True, 0),
                                                (16383, 256, 512, 1, False, 0), (16385, 300, 100, 0, True, 1),
                                                (20001, 256, 96, 1, False, 1), (16400, 768, 32, 1, True, 0)])
def test_b_split_once_gives_the_same_bits(m, n, k, tb, mask, beta):
    """With a workspace of qha_dense_project_workspace bytes, a product over at least 16384 rows of
    A splits B into its bf16 parts once per call instead of per tile; the bits must not change
    (same parts, same products, same order): ragged m, n and k, odd and single k-step counts, both
    storage orders of B, the ReLU mask, beta = 1, and a row count just below the threshold (no
    split, same bits trivially)."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng(m + n + k)
    a = rng.standard_normal((m, k)).astype(np.float32)
    b = (rng.standard_normal((n, k) if tb else (k, n)) / np.sqrt(k)).astype(np.float32)
    b[0, :7] = -0.0
    aux = np.where(rng.random((m, k)) < 0.5, -1.0, 1.0).astype(np.float32) if mask else None
    pro = B.PRO_RELU_MASK if mask else B.PRO_NONE
    ws_bytes = B.dense_project_workspace(0, tb, m, n, k)
    assert (ws_bytes > 0) == (m >= 16384)
    ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device="cuda")
    a_d, b_d = H.dev(a), H.dev(b)
    aux_d = H.dev(aux) if mask else None
    c0 = rng.standard_normal((m, n)).astype(np.float32)
    outs = []
    for w in (ws, None):
        H.note(f"b split once m={m} n={n} k={k} tb={tb} mask={mask} beta={beta} ws={w is not None}")
        c = H.dev(c0) if beta else torch.full((m, n), np.nan, dtype=torch.float32, device="cuda")
        B.dense_project(0, tb, a_d, b_d, beta, c, prologue=pro, aux=aux_d, workspace=w)
        outs.append(H.host(c))
    H.assert_bits_equal(outs[0], outs[1], "B split once against B split per tile")
    a64 = np.where(aux > 0, a, 0.0) if mask else a.astype(np.float64)
    b64 = b.astype(np.float64)
    ref = a64 @ (b64.T if tb else b64) + (c0.astype(np.float64) if beta else 0.0)
    H.assert_close(outs[0], ref, what="op(A) op(B)")


def test_backward_b_split_once_matches_dense_project():
    """qha_dense_backward at general widths: its dA (W split once into the workspace that dW's
    partials reuse afterwards) equals the per-tile split of qha_dense_project bit for bit."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    m, n, k = 20000, 256, 512
    rng = np.random.default_rng(7)
    a = rng.standard_normal((m, k)).astype(np.float32)
    w = (rng.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    h = np.where(rng.random((m, n)) < 0.5, 0.0, 1.0).astype(np.float32)
    dh = rng.standard_normal((m, n)).astype(np.float32)
    dh_d, h_d, a_d, w_d = H.dev(dh), H.dev(h), H.dev(a), H.dev(w)
    wsb = torch.empty(B.dense_backward_workspace(m, n, k) // 4 + 1, dtype=torch.float32, device="cuda")
    H.note("dense_backward dA against dense_project dA")
    da = torch.full((m, k), np.nan, dtype=torch.float32, device="cuda")
    dw = torch.full((n, k), np.nan, dtype=torch.float32, device="cuda")
    B.dense_backward(dh_d, h_d, a_d, w_d, da, dw, workspace=wsb)
    da2 = torch.full((m, k), np.nan, dtype=torch.float32, device="cuda")
    B.dense_project(0, 0, dh_d, w_d, 0, da2, prologue=B.PRO_RELU_MASK, aux=h_d)
    H.assert_bits_equal(H.host(da), H.host(da2), "dA")
    _, dw_ref = OD.project_backward(a, w, h, dh)
    H.assert_close_normwise(H.host(dw), dw_ref, what="dW after dA's use of the workspace")


def test_k_major_operand_beyond_2gib():
    """A k-major operand spanning more than 2 GiB (a 64-column slice of rows 16 KiB apart) is read
    with 64-bit addresses instead of 32-bit buffer offsets: the same bits as the contiguous copy,
    which takes the buffer loads, and the oracle's weight-gradient sum."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    m, n, k, ld = 140000, 16, 64, 4096
    assert m * ld * 4 >= 2 ** 31
    rng = np.random.default_rng(11)
    dz = rng.standard_normal((m, n)).astype(np.float32)
    a = rng.standard_normal((m, k)).astype(np.float32)
    H.note(f"k-major operand beyond 2 GiB: m={m} ld={ld}")
    big = torch.zeros((m, ld), dtype=torch.float32, device="cuda")
    big[:, :k] = H.dev(a)
    dz_d = H.dev(dz)
    outs = []
    for b_op in (big[:, :k], big[:, :k].contiguous()):
        ws = torch.empty(max(B.dense_project_workspace(1, 0, n, k, m), 16) // 4 + 4, dtype=torch.float32, device="cuda")
        c = torch.full((n, k), np.nan, dtype=torch.float32, device="cuda")
        B.dense_project(1, 0, dz_d, b_op, 0, c, workspace=ws)
        outs.append(H.host(c))
    del big
    H.assert_bits_equal(outs[0], outs[1], "strided beyond 2 GiB against contiguous")
    H.assert_close_normwise(outs[0], dz.astype(np.float64).T @ a.astype(np.float64), what="dZ^T A")


def _poisoned(rows, cols, data, device="cuda"):
    """data in the first `rows` rows of a buffer whose next rows hold NaN, returned as a view of
    those rows: a read past the operand's last row turns the result into NaN."""
    import torch
    buf = torch.full((rows + 8, cols), np.nan, dtype=torch.float32, device=device)
    buf[:rows] = H.dev(data)
    return buf[:rows]


@pytest.mark.parametrize("m,d_in,d_out", [(1001, 16, 16), (777, 256, 256), (4099, 512, 256), (3, 16, 16),
                                          (70001, 256, 256), (4098, 64, 512)])
def test_k_major_reduction_reads_nothing_past_its_rows(m, d_in, d_out):
    """dW = dZ^T A reduces over the m rows (k-major operands, m not a multiple of 4): the rows after
    dH, H and A hold NaN, and neither dW nor dA may see them (dense_project with trans_a = 1, and
    qha_dense_backward at general widths)."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    rng = np.random.default_rng(m + 5 * d_in + d_out)
    a = rng.standard_normal((m, d_in)).astype(np.float32)
    w = (rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)).astype(np.float32)
    h = OD.project(a, w).astype(np.float32)
    dh = rng.standard_normal((m, d_out)).astype(np.float32)
    da_ref, dw_ref = OD.project_backward(a, w, h, dh)
    dh_d, h_d, a_d = _poisoned(m, d_out, dh), _poisoned(m, d_out, h), _poisoned(m, d_in, a)
    w_d = H.dev(w)
    H.note(f"k-major ragged reduction m={m} {d_in}->{d_out}")
    ws_bytes = max(B.dense_project_workspace(1, 0, d_out, d_in, m), B.dense_backward_workspace(m, d_out, d_in))
    ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device="cuda")
    dw = torch.full((d_out, d_in), np.nan, dtype=torch.float32, device="cuda")
    B.dense_project(1, 0, dh_d, a_d, 0, dw, prologue=B.PRO_RELU_MASK, aux=h_d, workspace=ws)
    H.assert_close_normwise(H.host(dw), dw_ref, what="dW (dense_project, trans_a = 1)")
    # B stored k-major too (trans_b = 0): C = A^T A over the m rows
    c = torch.full((d_in, d_in), np.nan, dtype=torch.float32, device="cuda")
    ws2_bytes = B.dense_project_workspace(1, 0, d_in, d_in, m)
    ws2 = torch.empty(max(ws2_bytes // 4, 1), dtype=torch.float32, device="cuda")
    B.dense_project(1, 0, a_d, a_d, 0, c, workspace=ws2)
    a64 = a.astype(np.float64)
    H.assert_close_normwise(H.host(c), a64.T @ a64, what="A^T A")
    da = torch.full((m, d_in), np.nan, dtype=torch.float32, device="cuda")
    dw2 = torch.full((d_out, d_in), np.nan, dtype=torch.float32, device="cuda")
    B.dense_backward(dh_d, h_d, a_d, w_d, da, dw2, workspace=ws)
    H.assert_close(H.host(da), da_ref, what="dA (dense_backward)")
    H.assert_close_normwise(H.host(dw2), dw_ref, what="dW (dense_backward)")
