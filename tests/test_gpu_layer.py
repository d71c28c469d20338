"""Whole layers on the GPU (LayerStack, the bench's call sequence) against the oracle.

* Quantisation off (every halo at b = 32): the GPU stack and the oracle stack see identical inputs and
  make no random decisions, so outputs, embedding gradients and weight gradients are compared directly.
* Quantisation on: the stacks diverge wherever a float32 ulp moves a stochastic-rounding threshold,
  so each GPU call is fed the oracle's own intermediate inputs and compared with the oracle's next
  result (the oracle never consumes a GPU output).
"""
import dataclasses

import numpy as np
import pytest

import gpu_helpers as H
from oracle import layer as OL
from quantized_halo_aggregation_amd import synth

pytestmark = pytest.mark.gpu
SEED = synth.QUANT_SEED


def _stack(part):
    from quantized_halo_aggregation_amd.pipeline import GpuPartition, LayerStack
    gp = GpuPartition(part, chunk=64)
    return LayerStack(gp, part.weights, part.x, part.grad_top)


@pytest.mark.parametrize("model,layers,d,n_in", [("gcn", 3, 64, 700), ("gcn", 2, 128, 700), ("gcn", 2, 16, 701),
                                                  ("sage", 2, 64, 700)])
def test_unquantised_stack_matches_oracle(model, layers, d, n_in):
    """Every halo at b = 32: the stacks make no random decisions, so the GPU's outputs, embedding
    gradients and weight gradients are compared with the oracle's end to end, at the per-call rule
    (rtol 1e-5, atol 1e-6; dW norm-wise).  n_in = 701 makes the weight-gradient reductions run over a
    row count that is not a multiple of 4.

    GraphSAGE's embedding gradient dX = dA_self + mean^T(dA_mean) adds two products that cancel on
    some elements, and dA's own float32-class error (at most 8 units of 2^-24 of sum |dz w| per
    element, bounded by the dense error tests) then exceeds 1e-6 there.  Its check adds the error the
    chain can carry, 16 * 2^-24 * M, where M is the element's sum of absolute terms through the
    whole chain (the oracle run on |x|, |W|, |dH|)."""
    H.require_gpu()
    wl = synth.Workload(95, f"stack-{model}", n_in, 300, 9000, d, layers, model, ("const", 32))
    part = synth.make_partition(wl)
    fwds, bwds = OL.stack(part, SEED, 0)
    st = _stack(part)
    H.note(f"stack b=32 {model} L={layers} d={d} n_in={n_in}")
    st.step(epoch=0)
    slack = None
    if model == "sage":
        mag = dataclasses.replace(part, x=np.abs(part.x), weights=[np.abs(w) for w in part.weights],
                                  grad_top=np.abs(part.grad_top))
        _, mb = OL.stack(mag, SEED, 0)
        slack = [16 * 2.0 ** -24 * mb[l]["dx"].astype(np.float64) for l in range(layers)]
    for l in range(layers):
        H.assert_close(H.host(st.H[l]), fwds[l]["h"], what=f"H[{l}]")
        if slack is None:
            H.assert_close(H.host(st.dX[l]), bwds[l]["dx"], what=f"dX[{l}]")
        else:
            H.assert_close(H.host(st.dX[l]), bwds[l]["dx"], atol=1e-6 + slack[l], what=f"dX[{l}] (chained bound)")
        H.assert_close_normwise(H.host(st.dW[l]), bwds[l]["dw"], what=f"dW[{l}]")


def test_tiny_partition_layer_call_by_call():
    """The tiny workload (2,048 inner + 512 halo nodes, d = 16, widths from {1,2,4,8}): every call of the
    layer, forward and backward, fed with the oracle's inputs."""
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    part = synth.make_partition(synth.WORKLOADS[1])
    st = _stack(part)
    gp = st.gp
    n_in, d = part.n_in, part.d
    f = OL.gcn_forward(part, part.x, part.weights[0], 0, SEED, 0)
    b = OL.gcn_backward(part, f, part.weights[0], part.grad_top, 0, SEED, 0)
    H.note("tiny layer: quantize fwd")
    msg = gp.new_messages()
    gp.quantize_send(H.dev(part.x), gp.mirror, msg, 0, 0)
    H.assert_bits_equal(H.host(msg.codes).view(np.uint32)[:f["msg"]["words"].size], f["msg"]["words"], "codes fwd")
    H.assert_bits_equal(H.host(msg.scale), f["msg"]["scale"], "scale fwd")
    H.assert_bits_equal(H.host(msg.zero_point), f["msg"]["zero_point"], "zp fwd")
    H.note("tiny layer: aggregate fwd")
    a = torch.empty(n_in, d, dtype=torch.float32, device="cuda")
    gp.aggregate_fwd(H.dev(part.x), msg, a)
    from oracle import aggregate as OA
    x_cols = np.concatenate([part.x, f["msg"]["received"]])
    H.assert_close(H.host(a), OA.gcn_aggregate(part.nbr_ptr, part.nbr_idx, part.deg, x_cols), what="A")
    H.note("tiny layer: dense fwd")
    h = torch.empty(n_in, d, dtype=torch.float32, device="cuda")
    B.dense_project(0, 1, H.dev(f["a"]), H.dev(part.weights[0]), 0, h, epilogue=B.EPI_RELU)
    from oracle import dense as OD
    H.assert_close(H.host(h), OD.project(f["a"], part.weights[0]), what="H")
    H.note("tiny layer: dense bwd")
    da = torch.empty(n_in, d, dtype=torch.float32, device="cuda")
    dw = torch.empty(d, d, dtype=torch.float32, device="cuda")
    B.dense_project(0, 0, H.dev(part.grad_top), H.dev(part.weights[0]), 0, da, prologue=B.PRO_RELU_MASK,
                    aux=H.dev(f["h"]), workspace=st.dense_ws)
    B.dense_project(1, 0, H.dev(part.grad_top), H.dev(f["a"]), 0, dw, prologue=B.PRO_RELU_MASK,
                    aux=H.dev(f["h"]), workspace=st.dense_ws)
    da_ref, dw_ref = OD.project_backward(f["a"], part.weights[0], f["h"], part.grad_top)
    H.assert_close(H.host(da), da_ref, what="dA")
    H.assert_close_normwise(H.host(dw), dw_ref, what="dW")
    H.note("tiny layer: aggregate bwd + quantize bwd + received add")
    dxh = torch.empty(part.n_h, d, dtype=torch.float32, device="cuda")
    gp.aggregate_bwd_halo(H.dev(b["da"]), dxh)
    H.assert_close(H.host(dxh), OA.gcn_aggregate_t(part.nbr_ptr, part.nbr_idx, part.deg, b["da"])[n_in:], what="dX halo")
    msg_b = gp.new_messages()
    gp.quantize_send(H.dev(b["dx_cols"][n_in:]), None, msg_b, 0, 1)
    H.assert_bits_equal(H.host(msg_b.codes).view(np.uint32)[:b["msg"]["words"].size], b["msg"]["words"], "codes bwd")
    H.assert_bits_equal(H.host(msg_b.scale), b["msg"]["scale"], "scale bwd")
    dxi = torch.empty(n_in, d, dtype=torch.float32, device="cuda")
    gp.aggregate_bwd_inner(H.dev(b["da"]), dxi, 0)
    H.assert_close(H.host(dxi), b["dx_cols"][:n_in], rtol=1e-5, atol=1e-6, what="dX inner")
    dxi.copy_(H.dev(b["dx_cols"][:n_in]))
    gp.add_received(msg_b, dxi)
    H.assert_close(H.host(dxi), b["dx"], what="dX after received add")


def test_quantised_stack_runs_and_is_deterministic():
    """The quantised stack has no single right answer downstream of a rounding flip, but it must be
    deterministic and every quantised message must be a valid coding of its input (codes in range)."""
    H.require_gpu()
    part = synth.make_partition(synth.Workload(96, "stack-q", 900, 400, 12000, 128, 3, "gcn", ("top", 2, 4, 0.2)))
    st = _stack(part)
    H.note("quantised stack determinism")
    st.step(epoch=1)
    first = [H.host(t).copy() for t in st.H + st.dX + st.dW]
    st.step(epoch=1)
    second = [H.host(t) for t in st.H + st.dX + st.dW]
    for a, b in zip(first, second):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for t in first:
        assert np.isfinite(t).all()
