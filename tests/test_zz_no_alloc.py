"""qha_dequant_aggregate_fwd_noalloc: the aggregation without a workspace argument, whose split-row
partials go to the library's device scratch.  Called through the C ABI, it must give the bits of
qha_dequant_aggregate_fwd with a caller workspace on the same inputs (the same kernels run), and
match the oracle; two calls in a row, the second on a smaller partition, show that what the first
left in the scratch does not leak into the second."""
import numpy as np
import pytest

import gpu_helpers as H
from oracle import aggregate as OA
from quantized_halo_aggregation_amd import synth

pytestmark = pytest.mark.gpu
SEED = synth.QUANT_SEED


def _case(wl, chunk):
    from quantized_halo_aggregation_amd.pipeline import GpuPartition
    part = synth.make_partition(wl)
    gp = GpuPartition(part, chunk=chunk)
    assert gp.plan_fwd.struct.n_split_items > 0, "the case must split rows, so that the scratch is used"
    ref = H.oracle_messages(part.x[part.mirror], part.bits, SEED, 0, 0, part.n_in)
    return part, gp, ref, H.upload_messages(gp, ref)


def _noalloc(gp, x, msg, beta, out):
    from quantized_halo_aggregation_amd import binding as B
    lay = gp.layout
    B.dequant_aggregate_fwd_noalloc(gp.rowptr, gp.colidx, gp.w_fwd, gp.plan_fwd, x, gp.n_in, msg.codes,
                                    lay.word_offset, lay.bits, lay.classes, msg.meta, gp.n_h, beta, out)


def test_noalloc_aggregation_matches_the_workspace_call():
    H.require_gpu()
    import torch
    big = synth.Workload(91, "noalloc-big", 4000, 2000, 90_000, 128, 1, "gcn", ("top", 4, 8, 0.1))
    small = synth.Workload(92, "noalloc-small", 1200, 500, 20_000, 64, 1, "gcn", ("uniform", (1, 2, 4, 8)))
    for wl, beta in ((big, 0), (small, 1)):
        part, gp, ref, msg = _case(wl, chunk=32)
        n_in, d = part.n_in, part.d
        H.note(f"noalloc aggregation {wl.name} beta={beta} split items {gp.plan_fwd.struct.n_split_items}")
        x = H.dev(part.x)
        out0 = np.random.default_rng(wl.index).standard_normal((n_in, d)).astype(np.float32)
        got = H.dev(out0) if beta else torch.full((n_in, d), np.nan, dtype=torch.float32, device="cuda")
        _noalloc(gp, x, msg, beta, got)
        want = H.dev(out0) if beta else torch.full((n_in, d), np.nan, dtype=torch.float32, device="cuda")
        from quantized_halo_aggregation_amd import binding as B
        lay = gp.layout
        B.dequant_aggregate_fwd(gp.rowptr, gp.colidx, gp.w_fwd, gp.plan_fwd, x, n_in, msg.codes, lay.word_offset,
                                lay.bits, lay.classes, msg.meta, gp.n_h, beta, want, workspace=gp.agg_ws)
        H.assert_bits_equal(H.host(got), H.host(want), f"{wl.name}: noalloc vs workspace call")
        x_cols = np.concatenate([part.x, ref["received"]])
        oracle = OA.gcn_aggregate(part.nbr_ptr, part.nbr_idx, part.deg, x_cols) + (out0 if beta else 0)
        H.assert_close(H.host(got), oracle, what=f"{wl.name}: noalloc vs oracle")


def test_noalloc_aggregation_refuses_a_plan_beyond_its_scratch():
    H.require_gpu()
    import torch
    from quantized_halo_aggregation_amd import binding as B
    n_rows, row_len, d = 40, 40_000, 512
    ptr = np.arange(n_rows + 1, dtype=np.int32) * row_len
    plan = B.AggPlan(ptr, chunk=16)
    assert plan.workspace_bytes(d) > B.NOALLOC_SCRATCH_BYTES
    H.note("noalloc aggregation: plan beyond the scratch")
    col = torch.zeros(n_rows * row_len, dtype=torch.int32, device="cuda")
    x = torch.zeros(4, d, dtype=torch.float32, device="cuda")
    out = torch.zeros(n_rows, d, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="static scratch"):
        B.dequant_aggregate_fwd_noalloc(H.dev(ptr), col, None, plan, x, 4, None, None, None, None, None, 0, 0, out)
