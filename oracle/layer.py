"""One GPU's share of a GNN layer, forward and backward, chained from the oracle's pieces.

The per-layer data path of the SYLVIE guide (sections 5 and 11): the sender quantises each outgoing
boundary vector at that node's width, the exchange delivers codes and (min, scale), the receiver
dequantises and aggregates them with its local rows; the backward repeats this on embedding
gradients with the same per-node widths.

On one GPU the exchange is modelled by *mirrors*: halo node k is the remote copy of inner node
``mirror[k]``.  Forward, the vectors sent are the inner embeddings ``x[mirror]`` and the codes
received are the codes sent.  Backward, the gradients computed for the halo columns are quantised,
"sent" and added to the gradients of their mirror rows.  Random streams: stream id 2*layer for the
forward message, 2*layer + 1 for the backward one, node id n_in + k for halo k, so forward and
backward (and different layers) never share draws.

Each stage's output is rounded to float32, the training precision, before the next stage uses it.
"""
from __future__ import annotations

import numpy as np

from . import aggregate, dense, quantize


def _f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def send_halo(x_rows: np.ndarray, bits, seed, epoch, stream_id, node_base):
    """Quantise, pack and (on the receiving side) dequantise a block of boundary rows."""
    node_ids = node_base + np.arange(x_rows.shape[0], dtype=np.uint64)
    codes, scale, zp = quantize.stochastic_quantize(x_rows, bits, seed, epoch, stream_id, node_ids)
    words, off = quantize.pack(codes, bits)
    received = quantize.dequantize(codes, scale, zp, bits)
    return {"codes": codes, "words": words, "word_offset": off, "scale": scale, "zero_point": zp,
            "received": received}


def gcn_forward(part, x_inner, w, layer, seed, epoch):
    n_in = part.n_in
    msg = send_halo(x_inner[part.mirror], part.bits, seed, epoch, 2 * layer, n_in)
    x_cols = np.concatenate([x_inner, msg["received"]]).astype(np.float32)
    a = _f32(aggregate.gcn_aggregate(part.nbr_ptr, part.nbr_idx, part.deg, x_cols))
    h = _f32(dense.project(a, w))
    return {"msg": msg, "a": a, "h": h}


def gcn_backward(part, fwd, w, dh, layer, seed, epoch):
    n_in = part.n_in
    da, dw = dense.project_backward(fwd["a"], w, fwd["h"], dh)
    da = _f32(da)
    dx_cols = _f32(aggregate.gcn_aggregate_t(part.nbr_ptr, part.nbr_idx, part.deg, da))
    msg = send_halo(dx_cols[n_in:], part.bits, seed, epoch, 2 * layer + 1, n_in)
    dx_inner = _f32(aggregate.add_received(dx_cols[:n_in], part.mirror, msg["received"]))
    return {"da": da, "dw": dw, "dx_cols": dx_cols, "msg": msg, "dx": dx_inner}


def sage_forward(part, x_inner, w, layer, seed, epoch):
    n_in = part.n_in
    msg = send_halo(x_inner[part.mirror], part.bits, seed, epoch, 2 * layer, n_in)
    x_cols = np.concatenate([x_inner, msg["received"]]).astype(np.float32)
    m = _f32(aggregate.mean_aggregate(part.nbr_ptr, part.nbr_idx, x_cols))
    a = np.concatenate([x_inner, m], axis=1).astype(np.float32)
    h = _f32(dense.project(a, w))
    return {"msg": msg, "a": a, "h": h}


def sage_backward(part, fwd, w, dh, layer, seed, epoch):
    n_in, d = part.n_in, part.d
    da, dw = dense.project_backward(fwd["a"], w, fwd["h"], dh)
    da = _f32(da)
    n_cols = n_in + part.n_h
    dm = aggregate.mean_aggregate_t(part.nbr_ptr, part.nbr_idx, da[:, d:], n_cols)
    dx_cols = _f32(np.concatenate([da[:, :d].astype(np.float64) + dm[:n_in], dm[n_in:]]))
    msg = send_halo(dx_cols[n_in:], part.bits, seed, epoch, 2 * layer + 1, n_in)
    dx_inner = _f32(aggregate.add_received(dx_cols[:n_in], part.mirror, msg["received"]))
    return {"da": da, "dw": dw, "dx_cols": dx_cols, "msg": msg, "dx": dx_inner}


def stack(part, seed, epoch, n_layers=None):
    """Forward through every layer, then backward from ``part.grad_top``; returns per-layer records."""
    fwd_fn, bwd_fn = (sage_forward, sage_backward) if part.wl.model == "sage" else (gcn_forward, gcn_backward)
    n_layers = len(part.weights) if n_layers is None else n_layers
    x = part.x
    fwds = []
    for l in range(n_layers):
        f = fwd_fn(part, x, part.weights[l], l, seed, epoch)
        fwds.append(f)
        x = f["h"]
    g = part.grad_top
    bwds = [None] * n_layers
    for l in reversed(range(n_layers)):
        b = bwd_fn(part, fwds[l], part.weights[l], g, l, seed, epoch)
        bwds[l] = b
        g = b["dx"]
    return fwds, bwds
