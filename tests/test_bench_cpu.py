"""bench.py's host logic on the CPU: the one-GPU contract, the byte models (against hand counts on a
tiny CSR) and the lookup of counter traffic by kernel-source hash."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_row_words():
    # ceil(d * b / 32) words, d words for raw rows
    assert bench.row_words(128, [1, 2, 4, 8, 32]).tolist() == [4, 8, 16, 32, 128]
    assert bench.row_words(16, [1, 2, 4, 8, 32]).tolist() == [1, 1, 2, 4, 16]


# 3 rows over 4 inner + 2 halo columns, d = 4; halo 0 at 4 bits (1 word), halo 1 raw (4 words)
PTR = np.array([0, 2, 3, 5])
IDX = np.array([0, 4, 1, 1, 5])
HW = bench.row_words(4, [4, 32])


def test_per_edge_gather_bytes_by_hand():
    # edges: 5 x (index + weight) = 40; inner sources 0, 1, 1: 3 x 16 = 48; halo sources: words
    # (1 + 4) x 4 = 20 and two (min, scale) pairs = 16; rows: 3 x (bound 4 + 16 written) = 60
    assert bench.gather_bytes(PTR, IDX, 4, 4, HW, beta=0) == 40 + 48 + 20 + 16 + 60
    # beta = 1 reads each output row too; no weights drops 4 bytes an edge; row_ids adds 4 a row
    assert bench.gather_bytes(PTR, IDX, 4, 4, HW, beta=1) == 40 + 48 + 20 + 16 + 3 * (4 + 32)
    assert bench.gather_bytes(PTR, IDX, 4, 4, HW, beta=0, weighted=False) == 20 + 48 + 20 + 16 + 60
    assert bench.gather_bytes(PTR, IDX, 4, 4, HW, beta=0, row_ids=True) == 40 + 48 + 20 + 16 + 3 * 24


def test_compulsory_bytes_by_hand():
    # rowptr 16 + colidx 20 + six norms 24 + distinct inner rows {0, 1} 32 + distinct halo rows
    # {0, 1}: 20 of codes and 16 of (min, scale) + three output rows 48
    assert bench.compulsory_bytes(PTR, IDX, 4, 4, HW, 0, 6) == 16 + 20 + 24 + 32 + 36 + 48
    assert bench.compulsory_bytes(PTR, IDX, 4, 4, HW, 1, 6) == 16 + 20 + 24 + 32 + 36 + 96
    assert bench.compulsory_bytes(PTR, IDX, 4, 4, HW, 0, 6, row_ids=True) == 16 + 20 + 24 + 12 + 32 + 36 + 48
    # never more than the per-edge model, which reads a source once per edge
    assert bench.compulsory_bytes(PTR, IDX, 4, 4, HW, 0, 6) - 24 - 16 <= bench.gather_bytes(PTR, IDX, 4, 4, HW, 0)


def test_quantize_bytes_by_hand():
    # two rows of d = 4: 16 read + 8 (min, scale) + 4 row index each, codes 1 + 4 words
    assert bench.quantize_bytes(2, 4, [4, 32], gathered=True) == 2 * (16 + 8 + 4) + 4 * 5
    assert bench.quantize_bytes(2, 4, [4, 32], gathered=False) == 2 * (16 + 8) + 4 * 5


def test_counter_traffic_is_read_only_for_the_current_sources(monkeypatch):
    # every stage with kernel sources has a traffic line for the bench partition in profiles/
    for stage in ("quantize_fwd", "aggregate_fwd", "aggregate_bwd_quantize", "add_received"):
        got = bench.measured_traffic("gcn-300k-d128", stage)
        assert got is not None and got > 0, stage
    assert bench.measured_traffic("gcn-300k-d128", "no_such_stage") is None
    assert bench.measured_traffic("no-such-workload", "aggregate_fwd") is None
    # once a stage's sources change, its old counters no longer count
    monkeypatch.setattr(bench, "source_hash", lambda stage: "0" * 16)
    assert bench.measured_traffic("gcn-300k-d128", "aggregate_fwd") is None
