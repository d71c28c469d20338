"""Pins of the oracle's Philox4x32-10 (Salmon et al., SC'11) against something other than itself.

* PyTorch ships an independent, header-only Philox4x32-10 engine (ATen/core/PhiloxRNGEngine.h); a
  tiny C++ driver compiled here with g++ prints its output words for given counters and keys.
* Statistical checks: the 16-bit rounding thresholds are uniform and independent across node,
  feature group, epoch and stream.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


def _torch_include():
    try:
        import torch.utils.cpp_extension as ce
    except Exception:
        return None
    for p in ce.include_paths():
        if os.path.exists(os.path.join(p, "ATen", "core", "PhiloxRNGEngine.h")):
            return p
    return None


@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    inc = _torch_include()
    if inc is None or shutil.which("g++") is None:
        pytest.skip("PyTorch headers or g++ not available")
    exe = str(tmp_path_factory.mktemp("ptp") / "philox_torch_pin")
    subprocess.run(["g++", "-O1", "-std=c++17", f"-I{inc}",
                    os.path.join(HERE, "helpers", "philox_torch_pin.cpp"), "-o", exe], check=True)

    def run(rows):
        text = "\n".join(" ".join(str(int(v)) for v in r) for r in rows) + "\n"
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(t) for t in line.split()] for line in out.strip().splitlines()], dtype=np.uint64)

    return run


def test_philox_matches_pytorch_engine(torch_philox):
    rng = np.random.default_rng(7)
    rows = rng.integers(0, 2**32, size=(400, 6), dtype=np.uint64)
    rows[0] = 0
    rows[1] = 2**32 - 1
    rows[2, :4] = [5, 0, 1, 3]          # the (node, group, epoch, stream) shape of real use
    expect = torch_philox(rows)
    got = np.empty((rows.shape[0], 4), dtype=np.uint64)
    for i, r in enumerate(rows):
        w = philox.philox4x32([r[0]], [r[1]], [r[2]], [r[3]], int(r[4]), int(r[5]))
        got[i] = [int(x[0]) for x in w]
    np.testing.assert_array_equal(got, expect)


def test_threshold_layout_follows_generator_words():
    seed = 0x0123456789ABCDEF
    ids = np.array([3, 1000, 2**31 + 5], dtype=np.uint64)
    thr = philox.rounding_thresholds(ids, 24, seed, epoch=7, stream_id=2)
    for r, node in enumerate(ids):
        for g in range(3):
            w = philox.philox4x32([node], [g], [7], [2], seed & 0xFFFFFFFF, seed >> 32)
            for i in range(8):
                word = int(w[i // 2][0])
                half = word & 0xFFFF if i % 2 == 0 else word >> 16
                assert thr[r, 8 * g + i] == half


def test_thresholds_uniform_chi2():
    thr = philox.rounding_thresholds(np.arange(20000, dtype=np.uint64), 64, seed=11, epoch=0, stream_id=0)
    bins = np.bincount((thr >> 8).ravel(), minlength=256)
    expected = thr.size / 256
    chi2 = float(((bins - expected) ** 2 / expected).sum())
    # 255 degrees of freedom: mean 255, sd ~22.6; 6 sd margin
    assert chi2 < 255 + 6 * 22.6, chi2
    assert abs(thr.mean() / 65535.0 - 0.5) < 2e-3


@pytest.mark.parametrize("axis", ["node", "group", "epoch", "stream", "seed"])
def test_thresholds_independent_across_counter_fields(axis):
    n = 40000
    base = dict(node=np.arange(n, dtype=np.uint64), epoch=3, stream=1, seed=99)
    a = philox.rounding_thresholds(base["node"], 16, base["seed"], base["epoch"], base["stream"]).astype(np.float64)
    if axis == "node":
        b = philox.rounding_thresholds(base["node"] + 1, 16, 99, 3, 1).astype(np.float64)
    elif axis == "group":
        b = np.roll(a, -8, axis=1)      # group g+1 vs g of the same node
    elif axis == "epoch":
        b = philox.rounding_thresholds(base["node"], 16, 99, 4, 1).astype(np.float64)
    elif axis == "stream":
        b = philox.rounding_thresholds(base["node"], 16, 99, 3, 2).astype(np.float64)
    else:
        b = philox.rounding_thresholds(base["node"], 16, 100, 3, 1).astype(np.float64)
    x, y = a[:, :8].ravel(), b[:, :8].ravel()
    corr = np.corrcoef(x, y)[0, 1]
    assert abs(corr) < 5.0 / np.sqrt(x.size), corr
    assert not np.array_equal(a, b)
