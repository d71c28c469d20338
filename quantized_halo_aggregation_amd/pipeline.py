"""One GPU's share of a partition's GNN layers, driven through the C ABI.

The per-layer data path of the SYLVIE guide (sections 5 and 11) on one GPU:

  forward   quantize_pack(send set) -> [exchange] -> dequant_aggregate_fwd -> dense_project(+ReLU)
  backward  dense_backward(dA, dW; ReLU mask) -> aggregate_bwd(halo columns) then quantize_pack
            (or both in aggregate_bwd_quantize) -> [exchange] -> one dequant_aggregate_fwd over the
            inner columns' transposed rows plus the received messages of their halo copies (or
            aggregate_bwd, then a dequant_aggregate_fwd over the mirror map that adds them)

The exchange is the identity under the mirror model (halo k is the remote copy of inner node
mirror[k]): the codes sent are the codes received.  Everything numeric runs in libqha's kernels;
this module only lays out device buffers and issues the calls in order on one stream.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import binding as B
from . import synth

QUANT_SEED = synth.QUANT_SEED

# Shape of the aggregation work plans, a scheduling choice that the results do not depend on beyond
# the order in which float64 partials of a split row are added (measured on the five synthetic
# partitions): heavy rows are cut into chunks of 256 edges in the forward plans and 512 in the
# transposed ones, and short rows are grouped into items of at most 128 edges when items of 256 would
# leave fewer than four per wavefront slot of the chip (8 per SIMD, 1024 SIMDs), else 256.
PLAN_CHUNK_FWD = 256
PLAN_CHUNK_BWD = 512
PLAN_MIN_ITEMS = 4 * 8 * 1024


def plan_group_edges(rowptr, chunk: int) -> int:
    """The item edge budget of a plan over rowptr with the given chunk (see PLAN_MIN_ITEMS)."""
    return 128 if B.plan_items(rowptr, chunk, 256) < PLAN_MIN_ITEMS else 256


@dataclasses.dataclass
class Layout:
    """How the halo rows of a packed message buffer are laid out: per-row widths and word offsets,
    and the width classes when equal widths are contiguous (None: use the per-row arrays)."""
    h_bits: np.ndarray             # uint8 [n_h] (host)
    h_word_offset: np.ndarray      # uint32 [n_h + 1] (host)
    total_words: int
    bits: torch.Tensor             # the same two arrays on the device
    word_offset: torch.Tensor
    classes: object


@dataclasses.dataclass
class Messages:
    """One packed message buffer: the codes and per-row (min, scale) pairs of the halo rows, and the
    layout they were packed with (the receiver dequantises with the sender's widths, which matters
    when an asynchronous epoch reads messages packed at the previous epoch's widths)."""
    codes: torch.Tensor        # int32 words (uint32 bit patterns)
    meta: torch.Tensor         # float32 [n_h, 2]: min (zero-point), scale
    layout: Layout = None      # None: the partition's current layout

    @property
    def zero_point(self):
        return self.meta[:, 0]

    @property
    def scale(self):
        return self.meta[:, 1]


class GpuPartition:
    """Device-resident CSR / CSC / norms / widths / plans of one partition (set-up, untimed)."""

    def __init__(self, part: synth.Partition, device: str = "cuda", chunk: int = None, group_edges: int = None,
                 bits=None, chunk_bwd: int = None):
        self.part = part
        self.device = device
        n_in, n_h, d = part.n_in, part.n_h, part.d
        self.n_in, self.n_h, self.d = n_in, n_h, d
        self.n_cols = n_in + n_h
        self.model = part.wl.model
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)

        if self.model == "gcn":
            ptr, idx = synth.with_self_loops(part.nbr_ptr, part.nbr_idx)
        else:
            ptr, idx = part.nbr_ptr, part.nbr_idx
        self.h_ptr, self.h_idx = ptr, idx
        colptr, rowidx = B.csr_transpose(ptr, idx, self.n_cols)
        self.h_colptr, self.h_rowidx = colptr, rowidx
        self.rowptr, self.colidx = dev(ptr), dev(idx)
        self.colptr, self.rowidx = dev(colptr), dev(rowidx)

        # mirror map as a compact CSR: one row per inner node that has halo copies, listing them,
        # with row_ids naming the inner node
        m_ptr, m_idx = B.csr_transpose(np.arange(n_h + 1, dtype=np.int32), part.mirror, n_in)
        targets = np.flatnonzero(np.diff(m_ptr) > 0).astype(np.int32)
        mc_ptr = np.concatenate([[0], np.cumsum(np.diff(m_ptr)[targets])]).astype(np.int32)
        self.mirror = dev(part.mirror)
        self.m_ptr, self.m_idx, self.m_rows = dev(mc_ptr), dev(m_idx), dev(targets)
        self.h_m_ptr = mc_ptr
        # the same lists over every inner node (empty for nodes without copies): the received
        # messages the one-launch transposed gather adds as it stores the inner rows
        self.c_ptr = dev(m_ptr)

        self.set_bits(part.bits if bits is None else bits)

        # edge weights of the forward CSR and of its transpose (set-up kernels)
        self.deg = dev(part.deg)
        if self.model == "gcn":
            self.norm = torch.empty(self.n_cols, dtype=torch.float32, device=device)
            B.degree_norm(self.deg, B.NORM_GCN, self.norm)
            r_f, c_f, r_b, c_b = self.norm[:n_in], self.norm, self.norm, self.norm[:n_in]
        else:
            row_len = dev(np.diff(part.nbr_ptr).astype(np.int32))
            self.mean_r = torch.empty(n_in, dtype=torch.float32, device=device)
            B.degree_norm(row_len, B.NORM_MEAN, self.mean_r)
            r_f, c_f, r_b, c_b = self.mean_r, None, None, self.mean_r
        self.w_fwd = torch.empty(max(idx.size, 1), dtype=torch.float32, device=device)
        self.w_bwd = torch.empty(max(rowidx.size, 1), dtype=torch.float32, device=device)
        B.edge_weights(self.rowptr, self.colidx, r_f, c_f, self.w_fwd)
        B.edge_weights(self.colptr, self.rowidx, r_b, c_b, self.w_bwd)

        # the inner columns' transposed rows, each followed by the received halo messages of that
        # node's copies (halo ids n_in + k, weight 1): one dequantising gather then forms an inner
        # node's gradient and adds what its copies received (a6 inner range + a8)
        t_cnt = np.diff(colptr[:n_in + 1]).astype(np.int64)
        m_cnt = np.diff(m_ptr).astype(np.int64)
        r_ptr = np.concatenate([[0], np.cumsum(t_cnt + m_cnt)]).astype(np.int64)
        pos_t = np.repeat(r_ptr[:-1] - colptr[:n_in].astype(np.int64), t_cnt) + np.arange(int(colptr[n_in]))
        pos_m = np.repeat(r_ptr[:-1] + t_cnt - m_ptr[:-1].astype(np.int64), m_cnt) + np.arange(int(m_ptr[-1]))
        r_idx = np.empty(int(r_ptr[-1]), dtype=np.int32)
        r_idx[pos_t] = rowidx[:colptr[n_in]]
        r_idx[pos_m] = n_in + m_idx
        self.h_r_ptr, self.h_r_idx = r_ptr.astype(np.int32), r_idx
        self.r_ptr, self.r_idx = dev(self.h_r_ptr), dev(r_idx)
        self.w_recv = torch.ones(max(r_idx.size, 1), dtype=torch.float32, device=device)
        if pos_t.size:
            self.w_recv[torch.from_numpy(pos_t).to(device)] = self.w_bwd[:pos_t.size]

        # heavy rows are cut into chunks of `chunk` edges in the forward plans and `chunk_bwd` in the
        # transposed ones (by default PLAN_CHUNK_FWD / PLAN_CHUNK_BWD; an explicit chunk alone sets
        # both); items hold at most group_edges edges (by default plan_group_edges, per plan)
        if chunk_bwd is None:
            chunk_bwd = PLAN_CHUNK_BWD if chunk is None else chunk
        if chunk is None:
            chunk = PLAN_CHUNK_FWD
        self.chunk, self.chunk_bwd, self.group_edges = chunk, chunk_bwd, group_edges
        self.int_rows = None

        def mk(rp, c=chunk):
            g = plan_group_edges(rp, c) if group_edges is None else group_edges
            return B.AggPlan(rp, c, g, device=device)
        self.plan_fwd = mk(ptr)
        self.plan_bwd_halo = mk(colptr[n_in:], chunk_bwd)
        self.plan_bwd_inner = mk(colptr[:n_in + 1], chunk_bwd)
        self.plan_bwd_all = mk(colptr, chunk_bwd)
        self.plan_mirror = mk(mc_ptr)
        self.plan_recv = mk(self.h_r_ptr)
        ws = max(p.workspace_bytes(d) for p in (self.plan_fwd, self.plan_bwd_halo, self.plan_bwd_inner,
                                                 self.plan_bwd_all, self.plan_mirror, self.plan_recv))
        self.agg_ws = torch.empty(max(ws // 4, 4), dtype=torch.float32, device=device)
        self.dense_ws = None

    def split_interior(self):
        """Builds the interior / boundary split of the forward CSR (guide section 10: inner work runs
        while the boundary messages are produced): interior rows have no halo neighbour, so their
        aggregation needs no message.  Each part is a sub-CSR whose rows write out[row_ids]; their
        edge weights come from the same weight kernel, so every row's sum is the unsplit one."""
        if getattr(self, "int_rows", None) is not None:
            return
        ptr, idx, n_in = self.h_ptr, self.h_idx, self.n_in
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(self.device)
        cs = np.concatenate([[0], np.cumsum(idx >= n_in)])
        interior = (cs[ptr[1:]] - cs[ptr[:-1]]) == 0
        self.n_interior = int(interior.sum())

        def sub(rows):
            lens = np.diff(ptr)[rows].astype(np.int64)
            sptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            take = np.repeat(ptr[rows].astype(np.int64) - sptr[:-1], lens) + np.arange(int(sptr[-1]))
            sidx = idx[take]
            rows_d, sptr_d, sidx_d = dev(rows.astype(np.int32)), dev(sptr), dev(sidx)
            r = self.norm[rows_d.long()] if self.model == "gcn" else self.mean_r[rows_d.long()]
            c = self.norm if self.model == "gcn" else None
            w = torch.empty(max(sidx.size, 1), dtype=torch.float32, device=self.device)
            B.edge_weights(sptr_d, sidx_d, r.contiguous(), c, w)
            g = plan_group_edges(sptr, self.chunk) if self.group_edges is None else self.group_edges
            return rows_d, sptr_d, sidx_d, w, B.AggPlan(sptr, self.chunk, g, device=self.device)

        self.int_rows, self.int_ptr, self.int_idx, self.int_w, self.plan_int = sub(np.flatnonzero(interior))
        self.bnd_rows, self.bnd_ptr, self.bnd_idx, self.bnd_w, self.plan_bnd = sub(np.flatnonzero(~interior))
        ws = max(self.plan_int.workspace_bytes(self.d), self.plan_bnd.workspace_bytes(self.d))
        self.int_ws = torch.empty(max(ws // 4, 4), dtype=torch.float32, device=self.device)
        if ws > self.agg_ws.numel() * 4:
            self.agg_ws = torch.empty(ws // 4, dtype=torch.float32, device=self.device)

    def set_bits(self, bits, grouped: bool = True):
        """Per-halo widths of the messages quantised from now on.  If the halo rows are numbered so
        that equal widths are contiguous the packed buffers use the width-class layout (offsets by
        arithmetic); otherwise, or with grouped=False, the per-row offset table."""
        bits = np.ascontiguousarray(bits, dtype=np.uint8)
        off, total = B.pack_layout(bits, self.d)
        self.layout = Layout(bits, off, total, torch.from_numpy(bits).to(self.device),
                             torch.from_numpy(off.view(np.int32)).to(self.device),
                             B.pack_classes(bits, self.d) if grouped else None)

    # the current layout's arrays
    h_bits = property(lambda self: self.layout.h_bits)
    h_word_offset = property(lambda self: self.layout.h_word_offset)
    total_words = property(lambda self: self.layout.total_words)
    bits = property(lambda self: self.layout.bits)
    word_offset = property(lambda self: self.layout.word_offset)
    classes = property(lambda self: self.layout.classes)

    def words_at(self, max_bits: int) -> int:
        """Words of a buffer holding every halo row at max_bits (a bound for widths up to it)."""
        w = self.d if max_bits == 32 else (self.d * max_bits + 31) // 32
        return self.n_h * w

    def new_messages(self, capacity_words: int = 0) -> Messages:
        return Messages(torch.empty(max(self.total_words, capacity_words, 1), dtype=torch.int32, device=self.device),
                        torch.empty(self.n_h, 2, dtype=torch.float32, device=self.device))

    def _stamp(self, msg: Messages):
        lay = self.layout
        if msg.codes.numel() < lay.total_words:
            raise ValueError(f"message buffer of {msg.codes.numel()} words, the layout needs {lay.total_words}")
        msg.layout = lay
        return lay

    def dense_workspace(self, *shapes, backward=None):
        need = max(B.dense_project_workspace(*s) for s in shapes)
        if backward is not None:
            need = max(need, B.dense_backward_workspace(*backward))
        if need and (self.dense_ws is None or self.dense_ws.numel() * 4 < need):
            self.dense_ws = torch.empty(need // 4 + 4, dtype=torch.float32, device=self.device)
        return self.dense_ws

    # -------------------------------------------------------------------------------------
    # the calls of one layer
    # -------------------------------------------------------------------------------------

    def quantize_send(self, x, row_index, msg: Messages, epoch, stream_id, seed=QUANT_SEED):
        """a1 / a7: quantise the n_h outgoing boundary rows (x[row_index] or x itself) with the
        current widths."""
        lay = self._stamp(msg)
        B.quantize_pack(x, row_index, self.n_h, lay.bits, lay.word_offset, lay.classes, seed, epoch, stream_id,
                        self.n_in, msg.codes, msg.meta)

    def aggregate_fwd(self, x_inner, msg: Messages, out):
        """a3: out = sum over N(v) and v of w_vu * x~_u, halo rows dequantised from msg."""
        lay = msg.layout or self.layout
        B.dequant_aggregate_fwd(self.rowptr, self.colidx, self.w_fwd, self.plan_fwd, x_inner, self.n_in, msg.codes,
                                lay.word_offset, lay.bits, lay.classes, msg.meta, self.n_h, 0, out,
                                workspace=self.agg_ws)

    def aggregate_fwd_interior(self, x_inner, out):
        """a3 on the interior rows only (no message needed; split_interior() first)."""
        if self.n_interior:
            B.dequant_aggregate_fwd(self.int_ptr, self.int_idx, self.int_w, self.plan_int, x_inner, self.n_in, None,
                                    None, None, None, None, 0, 0, out, workspace=self.int_ws, row_ids=self.int_rows)

    def aggregate_fwd_boundary(self, x_inner, msg: Messages, out):
        """a3 on the boundary rows only, halo rows dequantised from msg."""
        lay = msg.layout or self.layout
        B.dequant_aggregate_fwd(self.bnd_ptr, self.bnd_idx, self.bnd_w, self.plan_bnd, x_inner, self.n_in, msg.codes,
                                lay.word_offset, lay.bits, lay.classes, msg.meta, self.n_h, 0, out,
                                workspace=self.agg_ws, row_ids=self.bnd_rows)

    def aggregate_bwd_all(self, grad_out, dx_cols):
        """a6 over every column in one launch: dx_cols [n_in + n_h, d] gets the inner columns'
        gradients in rows 0 .. n_in - 1 and the halo columns' after them (no tail between two
        launches; each row's sum is the same as in the two range calls)."""
        B.aggregate_bwd(self.colptr, self.rowidx, self.w_bwd, self.plan_bwd_all, grad_out, self.n_in, 0, dx_cols,
                        workspace=self.agg_ws)

    def aggregate_bwd_halo(self, grad_out, dx_halo):
        """a6 (halo range): gradients of the halo columns."""
        B.aggregate_bwd(self.colptr[self.n_in:], self.rowidx, self.w_bwd, self.plan_bwd_halo, grad_out, self.n_in, 0,
                        dx_halo, workspace=self.agg_ws)

    def aggregate_bwd_halo_quantize(self, grad_out, msg: Messages, epoch, stream_id, seed=QUANT_SEED,
                                    workspace=None):
        """a6 (halo range) + a7 fused: the halo columns' gradients, each quantised into msg as
        quantize_send would code it, without storing the gradient rows.  A call that may run
        concurrently with another aggregation needs a workspace of its own."""
        lay = self._stamp(msg)
        B.aggregate_bwd_quantize(self.colptr[self.n_in:], self.rowidx, self.w_bwd, self.plan_bwd_halo, grad_out,
                                 self.n_in, self.d, lay.bits, lay.word_offset, lay.classes, seed, epoch, stream_id,
                                 self.n_in, msg.codes, msg.meta,
                                 workspace=self.agg_ws if workspace is None else workspace)

    def aggregate_bwd_all_quantize(self, grad_out, dx_inner, msg: Messages, epoch, stream_id, beta,
                                   seed=QUANT_SEED, received: Messages = None):
        """a6 over every column + a7 in one launch: the inner columns' gradients into dx_inner (added
        to it when beta = 1), the halo columns' gradients quantised into msg as quantize_send would
        code them, without storing them.  With received (messages that arrived before the call, in
        their own layout), a8 too: each inner row gets its copies' dequantised messages added as it
        is stored, exactly as add_received would add them afterwards."""
        lay = self._stamp(msg)
        rcv = None
        if received is not None:
            rl = received.layout or self.layout
            rcv = (self.c_ptr, self.m_idx, self.n_h, received.codes, received.meta, rl.bits, rl.word_offset,
                   rl.classes)
        B.aggregate_bwd_quantize(self.colptr, self.rowidx, self.w_bwd, self.plan_bwd_all, grad_out, self.n_in, self.d,
                                 lay.bits, lay.word_offset, lay.classes, seed, epoch, stream_id, self.n_in, msg.codes,
                                 msg.meta, workspace=self.agg_ws, grad_in=dx_inner, n_stored=self.n_in, beta=beta,
                                 received=rcv)

    def aggregate_bwd_inner(self, grad_out, dx_inner, beta):
        """a6 (inner range): gradients of the inner columns (beta = 1 adds to dx_inner)."""
        B.aggregate_bwd(self.colptr[:self.n_in + 1], self.rowidx, self.w_bwd, self.plan_bwd_inner, grad_out,
                        self.n_in, beta, dx_inner, workspace=self.agg_ws)

    def aggregate_bwd_inner_received(self, grad_out, msg: Messages, dx_inner, beta):
        """a6 (inner range) + a8 in one gather: dx_inner (+)= the inner columns' transposed sums plus
        the dequantised gradient messages received for each inner node's halo copies."""
        lay = msg.layout or self.layout
        B.dequant_aggregate_fwd(self.r_ptr, self.r_idx, self.w_recv, self.plan_recv, grad_out, self.n_in, msg.codes,
                                lay.word_offset, lay.bits, lay.classes, msg.meta, self.n_h, beta, dx_inner,
                                workspace=self.agg_ws)

    def add_received(self, msg: Messages, dx_inner):
        """a8: dx_inner[mirror[k]] += dequantised gradient message k."""
        lay = msg.layout or self.layout
        B.dequant_aggregate_fwd(self.m_ptr, self.m_idx, None, self.plan_mirror, None, 0, msg.codes, lay.word_offset,
                                lay.bits, lay.classes, msg.meta, self.n_h, 1, dx_inner, workspace=self.agg_ws,
                                row_ids=self.m_rows)


class LayerStack:
    """Buffers and call order of a stack of GCN or GraphSAGE-mean layers on one partition.

    pipelined=True adds the guide's asynchronous execution mode (section 10): the halo messages of
    every layer and direction are double-buffered, and in an asynchronous epoch t the aggregations
    read the messages of epoch t-1 while the messages of epoch t are quantised on a second stream
    (so they overlap the compute stream's work) for use in epoch t+1.  Inner rows are always
    current; halo rows are one epoch stale.  A synchronous epoch quantises and then aggregates its
    own messages, as without pipelining.  Slot t % 2 holds epoch t's messages; both streams join at
    the end of every epoch, so no buffer is overwritten while it is still to be read.
    """

    def __init__(self, gp: GpuPartition, weights, x, grad_top, seed=QUANT_SEED, fused_halo_bwd: bool = False,
                 pipelined: bool = False, max_bits: int = 0, fold_received: bool = False,
                 split_interior: bool = False, recv_in_gather: bool = True):
        self.gp = gp
        self.seed = seed
        self.fused_halo_bwd = fused_halo_bwd
        # asynchronous epochs of the one-launch backward: the previous epoch's received messages are
        # added by that launch as it stores the inner rows (no separate received add)
        self.recv_in_gather = recv_in_gather
        self.fold_received = fold_received
        self.split_interior = split_interior
        if split_interior:
            gp.split_interior()
        self.pipelined = pipelined
        dev = gp.device
        n_in, d = gp.n_in, gp.d
        self.L = len(weights)
        self.W = [torch.from_numpy(w).to(dev) for w in weights]
        self.dW = [torch.empty_like(w) for w in self.W]
        sage = gp.model == "sage"
        self.sage = sage
        k_in = 2 * d if sage else d
        n_slots = 2 if pipelined else 1
        # message buffers sized for the current widths, or for any widths up to max_bits
        cap = gp.words_at(max_bits) if max_bits else 0
        words = max(gp.total_words, cap, 1)
        # Layer l's input rows and its forward messages share one allocation (and each layer's
        # backward messages another), so that the forward gather finds x, the codes and the
        # (min, scale) pairs within 4 GiB of one base and addresses them from it.
        xs = n_in * (k_in if sage else d)
        fwd = [self._arena([("x", xs)] + [(f"c{t}", words) for t in range(n_slots)] +
                           [(f"m{t}", 2 * gp.n_h) for t in range(n_slots)]) for _ in range(self.L)]
        bwd = [self._arena([(f"c{t}", words) for t in range(n_slots)] +
                           [(f"m{t}", 2 * gp.n_h) for t in range(n_slots)]) for _ in range(self.L)]
        msgs = lambda ar, t: Messages(ar[f"c{t}"].view(torch.int32), ar[f"m{t}"].view(gp.n_h, 2))
        self.msg_f = [[msgs(fwd[l], t) for t in range(n_slots)] for l in range(self.L)]
        self.msg_b = [[msgs(bwd[l], t) for t in range(n_slots)] for l in range(self.L)]
        # activations: A_l is layer l's aggregated input ([n, 2d] for SAGE with the self half
        # first), H_l its output.  For SAGE, H_{l-1} is the left half of A_l.
        if sage:
            self.A = [fwd[l]["x"].view(n_in, k_in) for l in range(self.L)]
            self.A[0][:, :d].copy_(torch.from_numpy(x).to(dev))
            self.H = [self.A[l + 1][:, :d] for l in range(self.L - 1)] + \
                     [torch.empty(n_in, d, dtype=torch.float32, device=dev)]
            self.X = [self.A[0][:, :d]] + self.H[:-1]
        else:
            self.A = [torch.empty(n_in, d, dtype=torch.float32, device=dev) for _ in range(self.L)]
            self.X = [fwd[l]["x"].view(n_in, d) for l in range(self.L)]
            self.X[0].copy_(torch.from_numpy(x).to(dev))
            self.H = self.X[1:] + [torch.empty(n_in, d, dtype=torch.float32, device=dev)]
        self.grad_top = torch.from_numpy(grad_top).to(dev)
        self.dA = [torch.empty(n_in, k_in, dtype=torch.float32, device=dev) for _ in range(self.L)]
        # GCN without the fused or folded halo paths runs its transposed aggregation as one launch
        # over all columns into [n_in + n_h, d]: the inner rows are dX, the halo rows the gradients
        # to quantise (one buffer per layer, since layer l's may still be quantised on the second
        # stream while layer l - 1 gathers).  The fused path (without the folded received add) runs
        # one launch over all columns too, coding the halo rows instead of storing them.
        self.one_bwd_gather = not sage and not fused_halo_bwd and not fold_received
        self.one_fused = fused_halo_bwd and not fold_received
        self.dX_cols = []
        if sage:
            # dL/dh of layer l's input rows = the self half of dA, plus the transposed mean (added
            # in place), plus the received halo gradients
            self.dX = [self.dA[l][:, :d] for l in range(self.L)]
        elif self.one_bwd_gather:
            self.dX_cols = [torch.empty(n_in + gp.n_h, d, dtype=torch.float32, device=dev) for _ in range(self.L)]
            self.dX = [c[:n_in] for c in self.dX_cols]
        else:
            self.dX = [torch.empty(n_in, d, dtype=torch.float32, device=dev) for _ in range(self.L)]
        # halo gradient rows before quantisation: one buffer, or one per layer when the quantisation
        # of layer l may still run on the second stream while layer l-1 gathers
        if self.one_bwd_gather:
            self.dX_halo = [c[n_in:] for c in self.dX_cols]
        else:
            n_halo_bufs = 0 if fused_halo_bwd else (self.L if pipelined else 1)
            self.dX_halo = [torch.empty(gp.n_h, d, dtype=torch.float32, device=dev) for _ in range(n_halo_bufs)]
        self.msg_epoch = [None] * n_slots          # epoch whose messages each slot holds
        self.comm = torch.cuda.Stream(device=dev) if (pipelined or split_interior) else None
        # split-row partials of the gather that runs on the second stream (the compute stream's
        # gathers keep using the partition's workspace meanwhile)
        self.comm_ws = torch.empty_like(gp.agg_ws) if (pipelined and fused_halo_bwd and not self.one_fused) else None
        self.dense_ws = gp.dense_workspace((0, 1, n_in, d, k_in), backward=(n_in, d, k_in))

    def _arena(self, parts):
        """One float32 allocation cut into named 1-D views (each at a 256-byte boundary)."""
        offs, total = [], 0
        for _, n in parts:
            offs.append(total)
            total += -(-n // 64) * 64
        buf = torch.empty(max(total, 64), dtype=torch.float32, device=self.gp.device)
        return {name: buf[o:o + n] for (name, n), o in zip(parts, offs)}

    def _on_comm(self, fn):
        """Runs fn on the second stream once the compute stream's work so far is done."""
        ready = torch.cuda.Event()
        ready.record(torch.cuda.current_stream())
        self.comm.wait_event(ready)
        with torch.cuda.stream(self.comm):
            fn()

    def forward_layer(self, l, epoch, hook=None, slot=0, sync=True):
        gp, d = self.gp, self.gp.d
        x = self.X[l]
        agg_out = self.A[l][:, d:] if self.sage else self.A[l]
        msg = self.msg_f[l][slot]
        if sync and self.split_interior:
            # interior rows on the second stream while the messages are quantised, then the rest
            self._on_comm(lambda: gp.aggregate_fwd_interior(x, agg_out))
            gp.quantize_send(x, gp.mirror, msg, epoch, 2 * l, self.seed)
            if hook: hook("quantize_fwd", l)
            gp.aggregate_fwd_boundary(x, msg, agg_out)
            torch.cuda.current_stream().wait_stream(self.comm)
        elif sync:
            gp.quantize_send(x, gp.mirror, msg, epoch, 2 * l, self.seed)
            if hook: hook("quantize_fwd", l)
            gp.aggregate_fwd(x, msg, agg_out)
        else:
            self._on_comm(lambda: gp.quantize_send(x, gp.mirror, msg, epoch, 2 * l, self.seed))
            gp.aggregate_fwd(x, self.msg_f[l][1 - slot], agg_out)
        if hook: hook("aggregate_fwd", l)
        B.dense_project(0, 1, self.A[l], self.W[l], 0, self.H[l], epilogue=B.EPI_RELU, workspace=self.dense_ws)
        if hook: hook("dense_fwd", l)

    def backward_layer(self, l, epoch, hook=None, slot=0, sync=True):
        gp, d = self.gp, self.gp.d
        dH = self.grad_top if l == self.L - 1 else self.dX[l + 1]
        B.dense_backward(dH, self.H[l], self.A[l], self.W[l], self.dA[l], self.dW[l], workspace=self.dense_ws)
        if hook: hook("dense_bwd", l)
        g = self.dA[l][:, d:] if self.sage else self.dA[l]
        msg = self.msg_b[l][slot]
        stream_id = 2 * l + 1
        beta = 1 if self.sage else 0
        if self.one_fused:
            # one launch over every column: the inner columns' gradients into dX (added to the self
            # half for SAGE), the halo columns' gradients coded into this epoch's message (it stays on
            # the compute stream in an asynchronous epoch too: its inner rows are needed next).  In an
            # asynchronous epoch the messages received are the previous epoch's, there before the
            # launch, so the launch adds them to the inner rows as it stores them.
            fold = not sync and self.recv_in_gather
            gp.aggregate_bwd_all_quantize(g, self.dX[l], msg, epoch, stream_id, beta, self.seed,
                                          received=self.msg_b[l][1 - slot] if fold else None)
            if hook: hook("aggregate_bwd_quantize_received" if fold else "aggregate_bwd_quantize", l)
            if fold:
                return
        elif self.fused_halo_bwd:
            send = lambda: gp.aggregate_bwd_halo_quantize(g, msg, epoch, stream_id, self.seed,
                                                          workspace=None if sync else self.comm_ws)
            if sync:
                send()
                if hook: hook("aggregate_bwd_halo_quantize", l)
            else:
                self._on_comm(send)
        else:
            buf = self.dX_halo[l if len(self.dX_halo) > 1 else 0]
            if self.one_bwd_gather:
                gp.aggregate_bwd_all(g, self.dX_cols[l])
                if hook: hook("aggregate_bwd", l)
            else:
                gp.aggregate_bwd_halo(g, buf)
                if hook: hook("aggregate_bwd_halo", l)
            send = lambda: gp.quantize_send(buf, None, msg, epoch, stream_id, self.seed)
            if sync:
                send()
                if hook: hook("quantize_bwd", l)
            else:
                self._on_comm(send)
        received = msg if sync else self.msg_b[l][1 - slot]
        if self.one_bwd_gather or self.one_fused:
            gp.add_received(received, self.dX[l])
            if hook: hook("add_received", l)
        elif self.fold_received:
            gp.aggregate_bwd_inner_received(g, received, self.dX[l], beta)
            if hook: hook("aggregate_bwd_inner_received", l)
        else:
            gp.aggregate_bwd_inner(g, self.dX[l], beta)
            if hook: hook("aggregate_bwd_inner", l)
            gp.add_received(received, self.dX[l])
            if hook: hook("add_received", l)

    def step(self, epoch=0, hook=None, sync=True):
        """One epoch: every layer forward, then backward.  sync=False (pipelined stacks only) runs the
        asynchronous mode, which needs the messages of epoch - 1."""
        slot = epoch % 2 if self.pipelined else 0
        if not sync:
            if not self.pipelined:
                raise ValueError("the asynchronous mode needs a pipelined stack")
            if self.msg_epoch[1 - slot] != epoch - 1:
                raise ValueError(f"epoch {epoch} cannot run asynchronously: the messages of epoch {epoch - 1} "
                                 "are not there (run it, synchronously or not, first)")
        for l in range(self.L):
            self.forward_layer(l, epoch, hook, slot, sync)
        for l in reversed(range(self.L)):
            self.backward_layer(l, epoch, hook, slot, sync)
        if not sync:
            torch.cuda.current_stream().wait_stream(self.comm)
        self.msg_epoch[slot] = epoch


class AdaptiveEpochs:
    """The online loop of the guide's section 11 on one GPU's share.  Each epoch runs with the node
    widths the Quant Orchestrator derives from the mask levels and the Coordinator's base width, in
    the execution mode the Coordinator chose; the epoch's partition losses and time then go to the
    Coordinator, which sets the base width and mode of the next epoch.  The stack must be pipelined
    (for asynchronous epochs) with message buffers for max_bits, and its halo nodes numbered by
    descending level (qha_level_order) so that every epoch's buffer stays grouped by width."""

    def __init__(self, stack: LayerStack, levels, coordinator, max_bits: int = 8):
        self.stack = stack
        self.levels = np.ascontiguousarray(levels, dtype=np.uint8)
        self.coordinator = coordinator
        self.max_bits = max_bits
        self.base = coordinator.state.bits
        self.sync = bool(coordinator.state.sync)
        self.t = 0

    def run_epoch(self):
        """Runs epoch t; returns (t, base width, synchronous, node widths)."""
        bits = B.node_bits(self.levels, self.base, self.max_bits)
        self.stack.gp.set_bits(bits)
        self.stack.step(epoch=self.t, sync=self.sync)
        return self.t, self.base, self.sync, bits

    def report(self, partition_losses, epoch_time: float):
        """The losses and time of the epoch just run: sets the next epoch's base width and mode."""
        self.base, self.sync = self.coordinator.step(partition_losses, epoch_time)
        self.t += 1

