#!/usr/bin/env python3
"""Throughput of one GPU's share of a quantised-halo GCN layer (forward + backward) on MI355X.

A step is one pass of the whole hot path over the 300k-inner + 150k-halo, d = 128 partition
(power-law in-degree, mean 25; halo widths 4 bits, 8 bits for the top 10% by degree):
quantise the send set, fused dequantise + aggregate, project + ReLU, project backward (dA and dW in
one pass), the transposed aggregate over every column with the halo columns' gradients quantised in
place (or, with --unfused-halo-bwd, stored and quantised by a second call), dequantise + add the
received gradients.

Prints one JSON line.  value = per-edge gather bytes of the quantise and aggregate calls of a step
(every edge reads its whole source row, no reuse assumed) divided by the whole step's wall time (the
dense projections are inside the timed step too).  Per-kernel times come from HIP events recorded on
the launch stream inside the timed steps; each kernel's roofline fraction is taken against its
compulsory bytes (each array once), a lower bound on its HBM traffic.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quant+aggregate GB/s (% HBM peak) and G edge·feat/s per layer at d=128"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0     # dense bf16 matrix cores
PARTS = 6                          # bf16 part products per float32 product (three-way split)


# ------------------------------------------------------------------------------------------------
# algorithmic bytes (what each call must move with no reuse assumed)
# ------------------------------------------------------------------------------------------------

def row_words(d, bits):
    bits = np.asarray(bits, dtype=np.int64)
    return np.where(bits == 32, d, (d * bits + 31) // 32)


def quantize_bytes(n_rows, d, bits, gathered):
    """Each row: read d floats (through the row index when gathered), write its packed codes and its
    (min, scale) pair.  Widths and offsets come from the width classes (no per-row table)."""
    w = row_words(d, bits)
    per_row = 4 * d + 8 + (4 if gathered else 0)
    return int(n_rows * per_row + 4 * w.sum())


def gather_quant_bytes(colptr, n_edges, d, halo_words):
    """The transposed gather over the halo columns with the quantisation fused in: every edge reads
    its row index, its weight and a d-float gradient row; every halo column reads its bound and
    writes its packed codes and (min, scale) instead of d floats."""
    n_rows = colptr.size - 1
    return int(n_edges * (8 + 4 * d) + n_rows * (4 + 8) + 4 * halo_words.sum())


def gather_bytes(rowptr, colidx, n_inner, d, halo_words, beta, weighted=True, row_ids=False):
    """Per-edge gather model: every edge reads its column index, its weight and a whole feature row
    (inner) or its packed code row plus (min, scale) (halo); every row reads its bound, writes d
    floats (and reads them first when beta = 1)."""
    n_rows = rowptr.size - 1
    e = colidx.size
    halo = colidx >= n_inner
    n_halo_e = int(halo.sum())
    edge = e * (4 + (4 if weighted else 0)) + (e - n_halo_e) * 4 * d
    if n_halo_e:
        k = colidx[halo] - n_inner
        edge += int(4 * halo_words[k].sum()) + n_halo_e * 8
    rows = n_rows * (4 + (4 if row_ids else 0) + 4 * d * (2 if beta else 1))
    return int(edge + rows)


def compulsory_bytes(rowptr, colidx, n_inner, d, halo_words, beta, n_norm, row_ids=False):
    """Each array a gather needs, once: the row bounds and column indices, one normalisation factor
    per node (the per-edge weights are derived from them), every distinct source row (a feature row,
    or a halo row's packed codes and (min, scale) pair) and the output rows (read too when beta = 1).
    A lower bound on the HBM traffic of the call."""
    n_rows = rowptr.size - 1
    cols = np.unique(colidx).astype(np.int64)
    inner = cols[cols < n_inner]
    halo = cols[cols >= n_inner] - n_inner
    src = inner.size * 4 * d + (int(4 * halo_words[halo].sum()) + 8 * halo.size if halo.size else 0)
    return int(4 * (n_rows + 1) + 4 * colidx.size + 4 * n_norm + (4 * n_rows if row_ids else 0) + src +
               4 * d * n_rows * (2 if beta else 1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first (the first few dozen steps after set-up run about 1%% slower)")
    ap.add_argument("--workload", type=int, default=2, help="synthetic partition index (2 = 300k-node d=128)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-async", action="store_true", help="skip timing the asynchronous (stale-halo) mode")
    ap.add_argument("--split-interior", action="store_true",
                    help="aggregate the interior rows (no halo neighbour) on a second stream while the send set "
                         "is quantised, then the boundary rows")
    ap.add_argument("--sweep-bits", action="store_true",
                    help="instead of the step line: one line with the step, quantise and aggregate times and "
                         "message bytes for every halo width in {1, 2, 4, 8, 32} on the chosen partition")
    ap.add_argument("--chunk", type=int, default=None)
    ap.add_argument("--chunk-bwd", type=int, default=None)
    ap.add_argument("--group-edges", type=int, default=None)
    ap.add_argument("--unfused-halo-bwd", action="store_true",
                    help="gather the halo columns' gradients into a buffer and quantise that, instead of coding "
                         "them inside the one-launch transposed gather (the default)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the multi-GPU exchange is not "
              "implemented here", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    from quantized_halo_aggregation_amd import synth
    fused = not args.unfused_halo_bwd
    wl = synth.WORKLOADS[args.workload]
    t0 = time.time()
    part = synth.make_partition(wl)
    gen_s = time.time() - t0
    print(f"[bench] generated {wl.describe()} in {gen_s:.1f}s", file=sys.stderr, flush=True)
    # the oracle's timings come first: its all-core run forks worker processes, which must happen
    # before this process touches the GPU
    cpu_times = None
    if not args.no_cpu_baseline and not args.sweep_bits:
        cpu_times = cpu_baseline_times(part)

    import torch
    from quantized_halo_aggregation_amd import binding as B
    from quantized_halo_aggregation_amd.pipeline import GpuPartition, LayerStack

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    gp = GpuPartition(part, chunk=args.chunk, chunk_bwd=args.chunk_bwd, group_edges=args.group_edges)
    st = LayerStack(gp, part.weights, part.x, part.grad_top, fused_halo_bwd=fused,
                    split_interior=args.split_interior)
    torch.cuda.synchronize()
    print("[bench] device set-up done", file=sys.stderr, flush=True)
    # the forward halo gather addresses the inner rows, codes and (min, scale) pairs from one base
    # when they lie within 4 GiB of each other
    m0 = st.msg_f[0][0]
    spans = [(st.X[0].data_ptr(), st.X[0].data_ptr() + st.X[0].stride(0) * st.X[0].shape[0] * 4),
             (m0.codes.data_ptr(), m0.codes.data_ptr() + m0.codes.numel() * 4),
             (m0.meta.data_ptr(), m0.meta.data_ptr() + m0.meta.numel() * 4)]
    span = max(h for _, h in spans) - min(l for l, _ in spans)
    print(f"[bench] forward gather buffers span {span / 2**20:.0f} MiB "
          f"({'one base' if span < 2**32 else 'separate bases'})", file=sys.stderr, flush=True)

    n_in, n_h, d = part.n_in, part.n_h, part.d
    if args.sweep_bits:
        sweep_bits(args, wl, part, gp)
        return
    hw = row_words(d, part.bits)
    nw = gp.h_colptr
    sage = wl.model == "sage"
    n_cols = n_in + n_h
    n_norm = n_cols if not sage else n_in        # GCN: one factor per node; SAGE: 1/|N(v)| per row
    # per-edge (gather) bytes and compulsory bytes per call of one layer
    b_q_fwd = quantize_bytes(n_h, d, part.bits, gathered=True)
    b_q_bwd = quantize_bytes(n_h, d, part.bits, gathered=False)
    inner_t, halo_t = (nw[:n_in + 1], gp.h_rowidx[:nw[n_in]]), (nw[n_in:] - nw[n_in], gp.h_rowidx[nw[n_in]:])
    bwd_beta = 1 if sage else 0
    edge = {"quantize_fwd": b_q_fwd, "quantize_bwd": b_q_bwd,
            "aggregate_fwd": gather_bytes(gp.h_ptr, gp.h_idx, n_in, d, hw, beta=0),
            "aggregate_bwd_inner": gather_bytes(*inner_t, 1 << 62, d, hw, beta=bwd_beta),
            "aggregate_bwd_halo": gather_bytes(*halo_t, 1 << 62, d, hw, beta=0),
            "add_received": gather_bytes(gp.h_m_ptr, np.arange(n_h), 0, d, hw, beta=1, weighted=False, row_ids=True),
            "aggregate_bwd_halo_quantize": gather_quant_bytes(nw[n_in:], int(nw[-1] - nw[n_in]), d, hw)}
    comp = {"quantize_fwd": b_q_fwd, "quantize_bwd": b_q_bwd,
            "aggregate_fwd": compulsory_bytes(gp.h_ptr, gp.h_idx, n_in, d, hw, 0, n_norm),
            "aggregate_bwd_inner": compulsory_bytes(*inner_t, 1 << 62, d, hw, bwd_beta, n_norm),
            "aggregate_bwd_halo": compulsory_bytes(*halo_t, 1 << 62, d, hw, 0, n_norm),
            "add_received": compulsory_bytes(gp.h_m_ptr, np.arange(n_h), 0, d, hw, 1, 0, row_ids=True)}
    # the fused halo path writes codes and (min, scale) pairs instead of the gradient rows
    comp["aggregate_bwd_halo_quantize"] = comp["aggregate_bwd_halo"] - 4 * d * n_h + int(4 * hw.sum()) + 8 * n_h
    # one launch over all columns: the two ranges together
    edge["aggregate_bwd"] = edge["aggregate_bwd_halo"] + edge["aggregate_bwd_inner"]
    comp["aggregate_bwd"] = compulsory_bytes(nw, gp.h_rowidx, 1 << 62, d, hw, 0, n_norm)
    # ... with the halo rows coded in place (codes and (min, scale) pairs written instead of the
    # rows) and, for SAGE, the inner rows added to dA's self half
    coded = int(4 * hw.sum()) + 8 * n_h - 4 * d * n_h + (4 * d * n_in if sage else 0)
    edge["aggregate_bwd_quantize"] = edge["aggregate_bwd"] + coded
    comp["aggregate_bwd_quantize"] = comp["aggregate_bwd"] + coded
    if fused:
        bwd = ["aggregate_bwd_quantize"]
    elif st.one_bwd_gather:
        bwd = ["aggregate_bwd", "quantize_bwd"]
    else:
        bwd = ["aggregate_bwd_halo", "quantize_bwd", "aggregate_bwd_inner"]
    byte_stages = ["quantize_fwd", "aggregate_fwd", *bwd, "add_received"]
    bytes_by_stage = {k: edge[k] for k in byte_stages}
    comp_by_stage = {k: comp[k] for k in byte_stages}
    k_in = 2 * d if sage else d
    flops_by_stage = {"dense_fwd": 2 * n_in * k_in * d, "dense_bwd": 4 * n_in * k_in * d}
    qa_bytes_step = wl.layers * sum(bytes_by_stage.values())
    edges_fwd = int(gp.h_idx.size)

    # ---- timing ------------------------------------------------------------------------------
    stream = torch.cuda.current_stream()
    stages = ["quantize_fwd", "aggregate_fwd", "dense_fwd", "dense_bwd", *bwd, "add_received"]
    events = []

    def hook(name, layer):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        events.append((name, ev))

    for w in range(args.warmup):
        st.step(epoch=w)
    torch.cuda.synchronize()
    print(f"[bench] {args.warmup} warm-up steps done", file=sys.stderr, flush=True)

    # the timed steps run bare; a second pass of as many steps records a HIP event on the launch
    # stream at every stage boundary (the events cost about 15 us per step, so they stay out of
    # the timed pass) and gives the per-stage times
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for s in range(args.steps):
        st.step(epoch=args.warmup + s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = wall * 1e3 / args.steps
    print(f"[bench] {args.steps} timed steps: {ms_per_step:.3f} ms/step wall", file=sys.stderr, flush=True)

    per_stage = {s: [] for s in stages}
    records = []
    torch.cuda.synchronize()
    inst0 = time.perf_counter()
    for s in range(args.steps):
        events.clear()
        first = torch.cuda.Event(enable_timing=True)
        first.record(stream)
        st.step(epoch=args.warmup + args.steps + s, hook=hook)
        prev = first
        for name, ev in events:
            records.append((name, prev, ev))
            prev = ev
    torch.cuda.synchronize()
    inst_ms_step = (time.perf_counter() - inst0) * 1e3 / args.steps
    for name, a, b in records:
        per_stage[name].append(a.elapsed_time(b))
    gpu_ms_step = sum(sum(v) for v in per_stage.values()) / args.steps
    print(f"[bench] {args.steps} instrumented steps: {inst_ms_step:.3f} ms/step wall, {gpu_ms_step:.3f} ms/step "
          "in stages (events)", file=sys.stderr, flush=True)

    # per-kernel averages (a stage appears once per layer per step)
    avg_ms = {s: float(np.mean(v)) for s, v in per_stage.items() if v}
    kernels = {}
    for s, ms in avg_ms.items():
        rec = {"avg_ms": round(ms, 5)}
        if s in bytes_by_stage:
            gbs = comp_by_stage[s] / (ms * 1e-3) / 1e9
            rec.update(bytes_compulsory=comp_by_stage[s], gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4),
                       bytes_per_edge_model=bytes_by_stage[s],
                       gather_gbs=round(bytes_by_stage[s] / (ms * 1e-3) / 1e9, 1))
        if s in flops_by_stage:
            # float32 products per second, and the bf16 part products the matrix cores ran
            tf = flops_by_stage[s] / (ms * 1e-3) / 1e12
            rec.update(flops=flops_by_stage[s], tflops=round(tf, 2), mfma_tflops=round(PARTS * tf, 1),
                       frac_mfma=round(PARTS * tf / BF16_MFMA_PEAK_TFLOPS, 4))
        kernels[s] = rec
    qa_ms = sum(avg_ms[s] for s in bytes_by_stage) * wl.layers
    value = qa_bytes_step / (ms_per_step * 1e-3) / 1e9
    kernel_qa_gbs = qa_bytes_step / (qa_ms * 1e-3) / 1e9
    gef_agg = edges_fwd * d / (avg_ms["aggregate_fwd"] * 1e-3) / 1e9
    gef_layer = edges_fwd * d * wl.layers / (ms_per_step * 1e-3) / 1e9

    # roofline of a stage (one call: the kernel, plus a short combine launch for split rows)
    def roofline_of(st_name):
        t = avg_ms[st_name]
        if st_name in bytes_by_stage:
            ach = comp_by_stage[st_name] / (t * 1e-3) / 1e9
            return {"kernel": st_name, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name, st_name),
                    "bytes": "compulsory (each array once, a lower bound on HBM traffic)",
                    "bytes_per_call": comp_by_stage[st_name],
                    "gather_gbs_per_edge_model": round(bytes_by_stage[st_name] / (t * 1e-3) / 1e9, 1),
                    "traffic_note": "rocprofv3 FETCH_SIZE + WRITE_SIZE per call, scaled by a plain copy; it counts "
                                    "the L2's requests to memory, including those the Infinity Cache serves",
                    "avg_us": round(t * 1e3, 1)}
        ach = PARTS * flops_by_stage[st_name] / (t * 1e-3) / 1e12     # bf16 part products
        return {"kernel": st_name, "bound": "mfma", "achieved": round(ach, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                "avg_us": round(t * 1e3, 1)}

    # the dominant stage is the longest one; the forward and transposed gathers, which take about as
    # long on the GCN partitions, are both reported under "rooflines"
    dom = max(avg_ms, key=avg_ms.get)
    roof = roofline_of(dom)
    rooflines = {st_name: roofline_of(st_name) for st_name in ("aggregate_fwd", "aggregate_bwd") if st_name in avg_ms}

    # the asynchronous mode (halo messages one epoch stale, quantised on a second stream): the same
    # partition and weights, epoch 0 synchronous, then asynchronous epochs
    async_rec = None
    if not args.no_async:
        def async_ms(recv_in_gather):
            ast = LayerStack(gp, part.weights, part.x, part.grad_top, fused_halo_bwd=fused, pipelined=True,
                             recv_in_gather=recv_in_gather)
            ast.step(epoch=0)
            for w in range(args.warmup):
                ast.step(epoch=1 + w, sync=False)
            torch.cuda.synchronize()
            a0 = time.perf_counter()
            for s_ in range(args.steps):
                ast.step(epoch=1 + args.warmup + s_, sync=False)
            torch.cuda.synchronize()
            return (time.perf_counter() - a0) * 1e3 / args.steps
        # with the one-launch backward, an asynchronous epoch adds the previous epoch's received
        # messages inside that launch; timed also with the separate received add
        a_ms = async_ms(True)
        a_sep = async_ms(False) if fused else None
        async_rec = {"ms_per_step": round(a_ms, 4), "value": round(qa_bytes_step / (a_ms * 1e-3) / 1e9, 1),
                     "vs_sync": round(ms_per_step / a_ms, 4),
                     "received_add": "in the one-launch transposed gather" if fused else "separate",
                     "ms_per_step_separate_received_add": None if a_sep is None else round(a_sep, 4)}
        print(f"[bench] asynchronous epochs: {a_ms:.3f} ms/step"
              + ("" if a_sep is None else f" ({a_sep:.3f} with the separate received add)"), file=sys.stderr,
              flush=True)

    copy_gbs = stream_copy_gbs()

    cpu = None
    if cpu_times is not None:
        cpu = cpu_baseline_record(cpu_times, qa_bytes_step)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "n_inner": n_in, "n_halo": n_h, "edges_with_self_loops": edges_fwd,
                   "d": d, "layers": wl.layers, "model": wl.model,
                   "halo_bits": {str(k): v for k, v in part.stats()["bits_hist"].items()},
                   "parallelism": "single-gpu"},
        "value_bytes": "per-edge gather model of the quantise and aggregate calls (every edge reads its whole "
                       "source row, no reuse assumed; it counts reads the caches serve, so it can exceed the HBM "
                       "peak), divided by the whole step's wall time",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "compulsory_gbs": round(wl.layers * sum(comp_by_stage.values()) / (ms_per_step * 1e-3) / 1e9, 1),
        "instrumented_pass": {"ms_per_step": round(inst_ms_step, 4), "stage_events_ms_per_step": round(gpu_ms_step, 4)},
        "kernel_quant_aggregate_gbs": round(kernel_qa_gbs, 1),
        "stream_copy": {"gbs": round(copy_gbs, 1), "value_pct": round(100 * value / copy_gbs, 2),
                        "kernel_quant_aggregate_pct": round(100 * kernel_qa_gbs / copy_gbs, 2)},
        "g_edge_feat_per_s": {"aggregate_fwd": round(gef_agg, 2), "full_layer": round(gef_layer, 2)},
        "quant_aggregate_bytes_per_step": qa_bytes_step,
        "message_bytes": {"main": int(4 * hw.sum()), "scales": 8 * n_h},
        "kernels": kernels,
        "roofline": roof,
        "rooflines": rooflines,
        "async_mode": async_rec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def sweep_bits(args, wl, part, gp):
    """The step at every uniform halo width (the guide's fixed-width ablation, section 14, and its
    Table XII split of message bytes into main data and scales), one JSON line."""
    import torch
    from quantized_halo_aggregation_amd.pipeline import LayerStack
    n_in, n_h, d = part.n_in, part.n_h, part.d
    stream = torch.cuda.current_stream()
    out = []
    for b in (1, 2, 4, 8, 32):
        bits = np.full(n_h, b, dtype=np.uint8)
        gp.set_bits(bits)
        st = LayerStack(gp, part.weights, part.x, part.grad_top)
        hw = row_words(d, bits)
        q_bytes = quantize_bytes(n_h, d, bits, gathered=True)
        a_bytes = gather_bytes(gp.h_ptr, gp.h_idx, n_in, d, hw, beta=0)
        per = {}
        recs = []

        def hook(name, layer):
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(stream)
            recs[-1].append((name, ev))

        for w in range(args.warmup):
            st.step(epoch=w)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s_ in range(args.steps):
            first = torch.cuda.Event(enable_timing=True)
            first.record(stream)
            recs.append([("", first)])
            st.step(epoch=args.warmup + s_, hook=hook)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        for r in recs:
            for (_, a), (name, e) in zip(r[:-1], r[1:]):
                per.setdefault(name, []).append(a.elapsed_time(e))
        qa = {k: float(np.mean(v)) for k, v in per.items() if k in ("quantize_fwd", "aggregate_fwd")}
        out.append({"bits": b, "ms_per_step": round(ms, 4),
                    "quantize_fwd_us": round(qa["quantize_fwd"] * 1e3, 1),
                    "aggregate_fwd_us": round(qa["aggregate_fwd"] * 1e3, 1),
                    "quant_aggregate_gbs": round((q_bytes + a_bytes) / ((qa["quantize_fwd"] + qa["aggregate_fwd"]) * 1e-3)
                                                 / 1e9, 1),
                    "message_main_MB": round(4 * hw.sum() / 1e6, 2),
                    "message_scales_MB": round((8 * n_h if b != 32 else 0) / 1e6, 2)})
        print(f"[bench] {b}-bit halos: {ms:.3f} ms/step", file=sys.stderr, flush=True)
        del st
    print(json.dumps({"metric": "per-width sweep", "workload": wl.name, "n_inner": n_in, "n_halo": n_h, "d": d,
                      "layers": wl.layers, "steps": args.steps, "warmup": args.warmup, "widths": out}))


# ------------------------------------------------------------------------------------------------
# measured HBM traffic (rocprofv3 FETCH_SIZE / WRITE_SIZE counters, scaled by a plain copy)
# ------------------------------------------------------------------------------------------------

KERNEL_SOURCES = {
    # the kernel source whose change invalidates a stage's counter reading
    "aggregate_fwd": ["csrc/gather.hip"],
    "aggregate_bwd_inner": ["csrc/gather.hip"],
    "aggregate_bwd": ["csrc/gather.hip"],
    "aggregate_bwd_quantize": ["csrc/gather.hip", "csrc/quant_common.hpp"],
    "quantize_fwd": ["csrc/quantize.hip", "csrc/quant_common.hpp"],
    "add_received": ["csrc/gather.hip"],
    "dense_fwd": ["csrc/gemm.hip", "csrc/panel.hip"],
    "dense_bwd": ["csrc/gemm.hip", "csrc/panel.hip"],
}


def source_hash(stage):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(stage, []):
        with open(os.path.join(ROOT, "quantized_halo_aggregation_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, stage):
    """HBM bytes per call of `stage`, from a `traffic` line in profiles/*.txt taken on the current
    kernel sources (None when there is none, or the sources have changed since)."""
    pdir = os.path.join(ROOT, "profiles")
    if stage not in KERNEL_SOURCES or not os.path.isdir(pdir):
        return None
    want = source_hash(stage)
    for name in sorted(os.listdir(pdir)):
        if not name.endswith(".txt"):
            continue
        with open(os.path.join(pdir, name)) as fh:
            for line in fh:
                f = line.split()
                if len(f) < 4 or f[0] != "traffic" or f[1] != workload or f[2] != stage:
                    continue
                kv = dict(x.split("=", 1) for x in f[3:] if "=" in x)
                if kv.get("src") == want and "bytes_per_call" in kv:
                    return int(kv["bytes_per_call"])
    return None


def stream_copy_gbs(mib=1024, reps=5):
    """A STREAM-style device copy on this GPU (read + write bytes per second), after the timed
    region: the practical streaming rate that the headline rates are also quoted against."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def calibrate_copy(mib):
    """A plain copy kernel of known size: reads and writes mib MiB per launch, five launches."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n * 4, "launches": 5}))


# ------------------------------------------------------------------------------------------------
# the oracle on the host cores (timed before the GPU is touched)
# ------------------------------------------------------------------------------------------------

_CPU = {}          # the partition, and per-stage buffers in memory shared with forked workers


def _blocks(n, k):
    edges = np.linspace(0, n, k + 1).astype(np.int64)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def _shared(shape, dtype):
    """An array in anonymous shared memory: worker processes forked after it write into it directly."""
    import mmap
    count = int(np.prod(shape))
    buf = mmap.mmap(-1, max(count * np.dtype(dtype).itemsize, 1))
    return np.frombuffer(buf, dtype=dtype, count=count).reshape(shape)


def _cpu_task(task):
    """One piece of a stage of the oracle's step: rows [a, b) of the stage's output, written in place."""
    from oracle import aggregate as OA
    from oracle import layer as OL
    from quantized_halo_aggregation_amd import synth
    kind, a, b = task
    c = _CPU
    part = c["part"]
    n_in = part.n_in
    rows = np.arange(a, b)
    gcn = part.wl.model == "gcn"
    if kind == "send_fwd":
        c["x_cols"][n_in + a:n_in + b] = OL.send_halo(part.x[part.mirror[a:b]], part.bits[a:b], synth.QUANT_SEED, 0,
                                                      0, n_in + a)["received"]
    elif kind == "aggregate_fwd":
        c["a"][a:b] = (OA.gcn_aggregate(part.nbr_ptr, part.nbr_idx, part.deg, c["x_cols"], rows=rows) if gcn else
                       OA.mean_aggregate(part.nbr_ptr, part.nbr_idx, c["x_cols"], rows=rows))
    elif kind == "aggregate_bwd":
        c["dx"][a:b] = (OA.gcn_aggregate_t(part.nbr_ptr, part.nbr_idx, part.deg, c["g"], cols=rows) if gcn else
                        OA.mean_aggregate_t(part.nbr_ptr, part.nbr_idx, c["g"], n_in + part.n_h, cols=rows))
    elif kind == "send_bwd":
        c["recv_b"][a:b] = OL.send_halo(c["dx"][n_in + a:n_in + b], part.bits[a:b], synth.QUANT_SEED, 0, 1,
                                        n_in + a)["received"]
    elif kind == "add_received":
        ks = np.flatnonzero((part.mirror >= a) & (part.mirror < b))
        c["dxi"][a:b] = OA.add_received(c["dx"][a:b], part.mirror[ks] - a, c["recv_b"][ks])
    else:
        raise ValueError(kind)


def _cpu_step(run):
    """The quantise and aggregate calls of one layer step, stage by stage; run(kind, n) computes the
    stage's n output rows (in row blocks)."""
    n_in, n_h = _CPU["part"].n_in, _CPU["part"].n_h
    run("send_fwd", n_h)
    run("aggregate_fwd", n_in)
    run("aggregate_bwd", n_in + n_h)
    run("send_bwd", n_h)
    run("add_received", n_in)


def _worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def cpu_baseline_times(part, repeats=3):
    """The oracle as it is, timed on the host on the quantise and aggregate calls of one full layer step
    of the same partition (send-set quantisation, forward aggregation, the transposed aggregation over
    every column, gradient quantisation and the received-gradient add): on one thread, then with the
    same calls split over row blocks across one worker process per core.  Median of `repeats` runs each."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits
    n_in, n_h, d = part.n_in, part.n_h, part.d
    _CPU.clear()
    _CPU.update(part=part, g=np.random.default_rng(7).standard_normal((n_in, d)).astype(np.float32),
                x_cols=_shared((n_in + n_h, d), np.float32), a=_shared((n_in, d), np.float64),
                dx=_shared((n_in + n_h, d), np.float32), recv_b=_shared((n_h, d), np.float32),
                dxi=_shared((n_in, d), np.float64))
    _CPU["x_cols"][:n_in] = part.x
    single = []
    with threadpool_limits(limits=1):
        for _ in range(repeats):
            t0 = time.perf_counter()
            _cpu_step(lambda kind, n: _cpu_task((kind, 0, n)))
            single.append(time.perf_counter() - t0)
    print(f"[bench] oracle, one thread: {np.median(single):.2f} s per step", file=sys.stderr, flush=True)
    cores = min(16, len(os.sched_getaffinity(0)))
    multi = []
    with mp.get_context("fork").Pool(cores, initializer=_worker_init) as pool:
        for _ in range(repeats):
            t0 = time.perf_counter()
            _cpu_step(lambda kind, n: pool.map(_cpu_task, [(kind, a, b) for a, b in _blocks(n, cores)], chunksize=1))
            multi.append(time.perf_counter() - t0)
    print(f"[bench] oracle, {cores} processes: {np.median(multi):.2f} s per step", file=sys.stderr, flush=True)
    _CPU.clear()
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "")
    except OSError:
        pass
    return {"single": sorted(single), "multi": sorted(multi), "cores": cores, "nproc": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_baseline_record(t, step_bytes):
    """The CPU figures in the unit of value: the same bytes of one step over the oracle's step time."""
    med_1, med_n = float(np.median(t["single"])), float(np.median(t["multi"]))
    return {"value": round(step_bytes / med_n / 1e9, 3), "unit": "GB/s", "cores": t["cores"], "kind": "oracle",
            "sample": f"the quantise and aggregate calls of one full layer step of the same partition "
                      f"({med_n:.2f} s with the calls split over row blocks across {t['cores']} worker processes, "
                      f"one thread each; median of {len(t['multi'])}); same bytes model as value",
            "seconds": [round(x, 3) for x in t["multi"]],
            "single_thread": {"value": round(step_bytes / med_1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "seconds": [round(x, 3) for x in t["single"]]},
            "nproc": t["nproc"], "affinity_cpus": t["affinity"], "cpu_model": t["cpu_model"]}


if __name__ == "__main__":
    main()
