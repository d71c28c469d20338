"""Shared helpers of the GPU parity tests (oracle on the CPU, libqha on the GPU, same seeded inputs)."""
import sys

import numpy as np
import pytest

try:
    import torch
except Exception:  # pragma: no cover
    torch = None


def require_gpu():
    if torch is None or not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from quantized_halo_aggregation_amd import binding  # noqa: F401  (fails loudly if not built)


def note(msg):
    """Names the case before a GPU step, so a failing run says what it was doing."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_close(got, ref, rtol=1e-5, atol=1e-6, what=""):
    """|got - ref| <= atol + rtol * |ref| element by element (ref in float64)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} elements out of tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} err {err[i]:.3e} bound {bound[i]:.3e}")


def assert_close_normwise(got, ref, rtol=1e-5, atol=1e-6, what=""):
    """|got - ref| <= atol + rtol * max|ref| element by element (for long reductions with cancellation)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref).max()
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert (err <= bound).all(), f"{what}: max err {err.max():.3e} > {bound:.3e}"


def assert_bits_equal(got, ref, what=""):
    got = np.ascontiguousarray(got)
    ref = np.ascontiguousarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    g = got.view(np.uint32) if got.dtype.itemsize == 4 else got
    r = ref.view(np.uint32) if ref.dtype.itemsize == 4 else ref
    if not np.array_equal(g, r):
        bad = np.flatnonzero(g.ravel() != r.ravel())
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first at {bad[0]}: "
                             f"got {g.ravel()[bad[0]]:#x} ref {r.ravel()[bad[0]]:#x}")


def oracle_messages(x_rows, bits, seed, epoch, stream_id, node_base):
    """The oracle's packed messages for a block of rows (words, offsets, scale, zp, dequantised)."""
    from oracle import layer as OL
    return OL.send_halo(x_rows, np.asarray(bits), seed, epoch, stream_id, node_base)


def upload_messages(gp, msg):
    from quantized_halo_aggregation_amd.pipeline import Messages
    assert np.array_equal(msg["word_offset"], gp.h_word_offset.astype(np.int64))
    words = msg["words"] if msg["words"].size else np.zeros(1, np.uint32)
    meta = np.stack([msg["zero_point"], msg["scale"]], axis=1).astype(np.float32)
    return Messages(dev(words.view(np.int32)), dev(meta))
