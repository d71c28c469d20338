"""The asynchronous execution mode (SYLVIE guide, section 10; the epoch-tag checks of section 16):
in an asynchronous epoch the inner rows are current while the halo rows, forward and backward, come
from the previous epoch's messages, and the epoch's own messages are produced on a second stream for
the next one.  Checked against the oracle with the previous epoch's inputs put in by hand."""
import dataclasses

import numpy as np
import pytest

import gpu_helpers as H
from oracle import aggregate as OA
from oracle import dense as OD
from oracle import layer as OL
from quantized_halo_aggregation_amd import synth

pytestmark = pytest.mark.gpu
SEED = synth.QUANT_SEED


def _f32(a):
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def _stack(part, fused=False):
    from quantized_halo_aggregation_amd.pipeline import GpuPartition, LayerStack
    gp = GpuPartition(part, chunk=64)
    return LayerStack(gp, part.weights, part.x, part.grad_top, fused_halo_bwd=fused, pipelined=True)


@pytest.mark.parametrize("fused", [False, True], ids=["gather+quantize", "fused"])
def test_async_epoch_uses_previous_halo_messages_unquantised(fused):
    """All halos at b = 32 (no random decisions): epoch 0 synchronous on x0, epoch 1 asynchronous on
    x1; every layer of epoch 1 must equal the oracle chain whose halo columns carry epoch 0's
    embeddings (forward) and epoch 0's halo gradients (backward)."""
    H.require_gpu()
    wl = synth.Workload(97, "async-b32", 700, 300, 9000, 64, 2, "gcn", ("const", 32))
    part = synth.make_partition(wl)
    n_in, L = part.n_in, wl.layers
    x0 = part.x
    x1 = np.random.default_rng(1).standard_normal(x0.shape).astype(np.float32)
    fw0, bw0 = OL.stack(part, SEED, 0)                 # the synchronous epoch 0, fresh messages
    st = _stack(part, fused)
    H.note(f"async b=32 epoch 0 sync (fused={fused})")
    st.step(epoch=0)
    st.X[0].copy_(H.dev(x1))
    H.note("async b=32 epoch 1 async")
    st.step(epoch=1, sync=False)

    # oracle chain of epoch 1 with stale halo rows
    x_prev = [x0] + [fw0[l]["h"] for l in range(L - 1)]
    xs, fw1 = x1, []
    for l in range(L):
        x_cols = np.concatenate([xs, x_prev[l][part.mirror]])
        a = _f32(OA.gcn_aggregate(part.nbr_ptr, part.nbr_idx, part.deg, x_cols))
        h = _f32(OD.project(a, part.weights[l]))
        fw1.append({"a": a, "h": h})
        xs = h
    dh = part.grad_top
    for l in reversed(range(L)):
        da, dw = OD.project_backward(fw1[l]["a"], part.weights[l], fw1[l]["h"], dh)
        da = _f32(da)
        dx_cols = _f32(OA.gcn_aggregate_t(part.nbr_ptr, part.nbr_idx, part.deg, da))
        stale_halo = bw0[l]["dx_cols"][n_in:]
        dx = _f32(OA.add_received(dx_cols[:n_in], part.mirror, stale_halo))
        H.assert_close(H.host(st.H[l]), fw1[l]["h"], what=f"H[{l}] epoch 1")
        H.assert_close(H.host(st.dX[l]), dx, what=f"dX[{l}] epoch 1")
        H.assert_close_normwise(H.host(st.dW[l]), dw, what=f"dW[{l}] epoch 1")
        # epoch 1's own messages wait in slot 1 for epoch 2 (raw rows at b = 32)
        got = H.host(st.msg_b[l][1].codes).view(np.float32)[:part.n_h * part.d].reshape(part.n_h, part.d)
        H.assert_close(got, dx_cols[n_in:], what=f"epoch 1 halo gradients [{l}]")
        dh = dx


@pytest.mark.parametrize("fused", [False, True], ids=["gather+quantize", "fused"])
def test_epoch_tags_of_quantised_messages(fused):
    """Quantised halos (4 bits, top 10% at 8): the first layer's aggregation of an asynchronous epoch
    dequantises the codes quantised in the previous epoch (their epoch tag is in the rounding draws),
    the epoch's own codes go to the other slot untouched by the aggregation, and a synchronous epoch
    after it is fresh again; an asynchronous epoch without its predecessor's messages is refused."""
    H.require_gpu()
    import torch
    part = synth.make_partition(synth.Workload(98, "async-q", 1500, 600, 20000, 128, 1, "gcn", ("top", 4, 8, 0.1)))
    n_in, d = part.n_in, part.d
    xs = [np.random.default_rng(10 + e).standard_normal((n_in, d)).astype(np.float32) for e in range(3)]
    st = _stack(part, fused)
    gp = st.gp

    def check_aggregate(x_inner, msg_ref, what):
        x_cols = np.concatenate([x_inner, msg_ref["received"]])
        H.assert_close(H.host(st.A[0]), OA.gcn_aggregate(part.nbr_ptr, part.nbr_idx, part.deg, x_cols), what=what)

    def check_message(slot, x_rows, epoch, what):
        ref = OL.send_halo(x_rows, part.bits, SEED, epoch, 0, n_in)
        m = st.msg_f[0][slot]
        H.assert_bits_equal(H.host(m.codes).view(np.uint32)[:ref["words"].size], ref["words"], what + " codes")
        H.assert_bits_equal(H.host(m.meta), np.stack([ref["zero_point"], ref["scale"]], 1), what + " meta")
        return ref

    H.note(f"epoch tags: epoch 0 synchronous (fused={fused})")
    st.X[0].copy_(H.dev(xs[0]))
    st.step(epoch=0)
    m0 = check_message(0, xs[0][part.mirror], 0, "epoch 0")
    check_aggregate(xs[0], m0, "epoch 0 aggregate (fresh)")

    H.note("epoch tags: epoch 1 asynchronous")
    st.X[0].copy_(H.dev(xs[1]))
    st.step(epoch=1, sync=False)
    check_aggregate(xs[1], m0, "epoch 1 aggregate (inner current, halos from epoch 0)")
    check_message(1, xs[1][part.mirror], 1, "epoch 1 (produced for epoch 2)")
    check_message(0, xs[0][part.mirror], 0, "epoch 0 (kept)")

    H.note("epoch tags: epoch 2 synchronous")
    st.X[0].copy_(H.dev(xs[2]))
    st.step(epoch=2)
    m2 = check_message(0, xs[2][part.mirror], 2, "epoch 2")
    check_aggregate(xs[2], m2, "epoch 2 aggregate (fresh again)")
    with pytest.raises(ValueError):
        st.step(epoch=4, sync=False)
    # an asynchronous epoch gives the same result every time it is replayed from the same state
    st.step(epoch=3, sync=False)
    first = [H.host(t).copy() for t in (st.H[0], st.dX[0], st.dW[0])]
    st.step(epoch=2)
    st.step(epoch=3, sync=False)
    for a, b in zip(first, (st.H[0], st.dX[0], st.dW[0])):
        assert np.array_equal(a.view(np.uint32), H.host(b).view(np.uint32))
    torch.cuda.synchronize()


def test_adaptive_epochs_follow_the_coordinator():
    """The online loop (guide section 11): per epoch the Coordinator's base width and mode, the Quant
    Orchestrator's node widths on a partition numbered by the Graph Extractor's levels, and an
    asynchronous epoch that changes the widths still dequantises the previous epoch's messages with
    the widths they were packed with.  Every epoch's first-layer aggregation is checked against the
    oracle fed with the right epoch's inputs and widths."""
    H.require_gpu()
    from oracle import control as OC
    from quantized_halo_aggregation_amd import binding as B
    from quantized_halo_aggregation_amd.pipeline import AdaptiveEpochs, GpuPartition, LayerStack
    from test_oracle_control import LITERAL, TRACE

    part0 = synth.make_partition(synth.small_workload(1500, 700, 20000, 128, bits=("const", 4), index=94))
    n_in, d = part0.n_in, part0.d
    lv0 = OC.mask_levels(part0.deg[n_in:])
    ptr, idx, deg, mirror, lv = synth.number_halos_by_width(n_in, part0.nbr_ptr, part0.nbr_idx, part0.deg,
                                                            part0.mirror, lv0)
    part = dataclasses.replace(part0, nbr_ptr=ptr, nbr_idx=idx, deg=deg, mirror=mirror,
                               bits=OC.combine_and_clip(lv, 1))
    gp = GpuPartition(part)
    st = LayerStack(gp, part.weights, part.x, part.grad_top, pipelined=True, max_bits=8)
    run = AdaptiveEpochs(st, B.mask_levels(deg[n_in:])[0], B.Coordinator(lam=0.0, delta=2))
    xs = [np.random.default_rng(40 + t).standard_normal((n_in, d)).astype(np.float32) for t in range(len(TRACE))]
    want = [(1, True)] + LITERAL[:-1]            # the mode of epoch t is the decision after epoch t - 1
    used = {}
    for t, loss in enumerate(TRACE):
        H.note(f"adaptive epoch {t}: expect base {want[t][0]}, sync {want[t][1]}")
        st.X[0].copy_(H.dev(xs[t]))
        t_run, base, sync, bits = run.run_epoch()
        assert (t_run, base, sync) == (t, *want[t])
        assert np.array_equal(bits, OC.combine_and_clip(lv, base))
        used[t] = base
        src = t if sync else t - 1
        ref = OL.send_halo(xs[src][mirror], OC.combine_and_clip(lv, used[src]), SEED, src, 0, n_in)
        x_cols = np.concatenate([xs[t], ref["received"]])
        H.assert_close(H.host(st.A[0]), OA.gcn_aggregate(ptr, idx, deg, x_cols),
                       what=f"epoch {t} aggregate (halos of epoch {src} at base {used[src]})")
        run.report([loss], 1.0)


@pytest.mark.parametrize("d", [64, 128])
def test_interior_split_gives_the_unsplit_result(d):
    """The interior / boundary split (interior rows aggregated on the second stream while the messages
    are quantised) changes no row's arithmetic: every output of a synchronous step equals the unsplit
    step's bit for bit, and the interior rows really have no halo neighbour."""
    H.require_gpu()
    from quantized_halo_aggregation_amd.pipeline import GpuPartition, LayerStack
    part = synth.make_partition(synth.small_workload(4000, 150, 24000, d, bits=("top", 4, 8, 0.1), index=91))
    n_in = part.n_in
    outs = []
    for split in (False, True):
        gp = GpuPartition(part, chunk=64)
        st = LayerStack(gp, part.weights, part.x, part.grad_top, split_interior=split)
        H.note(f"interior split={split} d={d}")
        st.step(epoch=2)
        outs.append([H.host(t).copy() for t in (st.A[0], st.H[0], st.dX[0], st.dW[0])])
        if split:
            rows = H.host(gp.int_rows).astype(np.int64)
            assert gp.n_interior == rows.size and 0.2 * n_in < rows.size < n_in
            for r in rows[:200]:
                assert np.all(part.nbr_idx[part.nbr_ptr[r]:part.nbr_ptr[r + 1]] < n_in)
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("model", ["gcn", "sage"])
def test_async_received_add_in_the_gather_changes_nothing(model):
    """In an asynchronous epoch the one-launch transposed gather adds the previous epoch's received
    messages as it stores the inner rows; the epoch's every output (H, dX, dW and the messages it
    codes, forward and backward) equals, bit for bit, the same epoch with the separate received add."""
    H.require_gpu()
    from quantized_halo_aggregation_amd.pipeline import GpuPartition, LayerStack
    part = synth.make_partition(synth.Workload(96, f"async-fold-{model}", 1200, 700, 16000, 128, 2, model,
                                               ("top", 4, 8, 0.1)))
    outs = []
    for fold in (True, False):
        gp = GpuPartition(part, chunk=64)
        st = LayerStack(gp, part.weights, part.x, part.grad_top, fused_halo_bwd=True, pipelined=True,
                        recv_in_gather=fold)
        H.note(f"async received add in the gather={fold} ({model})")
        seen = []
        st.step(epoch=0)
        st.step(epoch=1, sync=False, hook=lambda name, l: seen.append(name))
        assert ("aggregate_bwd_quantize_received" in seen) == fold and ("add_received" in seen) != fold
        outs.append([H.host(t).copy() for l in range(st.L)
                     for t in (st.H[l], st.dX[l], st.dW[l], st.msg_f[l][1].codes, st.msg_f[l][1].meta,
                               st.msg_b[l][1].codes, st.msg_b[l][1].meta)])
    for i, (a, b) in enumerate(zip(*outs)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"output {i} differs"
