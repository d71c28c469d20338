"""Stochastic integer quantisation of boundary messages (SYLVIE guide, section 6), in float32.

For one message vector h of D features and a width b in {1, 2, 4, 8}:
  scale = (max h - min h) / (2^b - 1);   q = stochastic_round((h - min h) / scale);
  received value = scale * q + min h     (min h is the zero-point).
Stochastic rounding takes the upper neighbour with probability equal to the fractional part, so
the dequantised value is unbiased; its variance grows with scale^2.  Only messages crossing the
partition boundary are quantised; b = 32 marks a message sent as raw float32 (the guide's "b=32"
ablation setting).

Floating-point steps are fixed so that two implementations give identical integers:
  mn, mx      exact min and max;  zero_point = mn + 0 (turns -0 into +0)
  range       fl(mx - mn);  range == 0 -> scale 0, every code 0 (the zero-scale boundary); the
              same when fl(L / range) overflows (range below L / FLT_MAX, about 7.5e-37 at b = 8)
  scale       fl(range / L) with L = 2^b - 1 (correctly rounded division)
  inv         fl(L / range)
  y           fl(fl(h - mn) * inv)    -- a multiply by the reciprocal instead of a division per
                                         element; the two differ by at most one ulp of y
  f, fr       floor(y), y - f (exact)
  up          u < fr * 2^16 for the 16-bit uniform threshold u of this element
  q           min(f + up, L)
With a 16-bit threshold, P(up) = ceil(fr * 2^16) / 2^16, a bias below 2^-16 * scale.

Packing: row r occupies ceil(D*b/32) 32-bit words (D words when b = 32); the code of feature j sits
at bit j*b, least significant bit first, unused high bits are zero.  Rows follow each other in the
caller's order starting at word_offset[r] (an exclusive prefix sum of the row sizes); grouping the
send buffer by width, as the guide suggests, is just a different row order.
"""
from __future__ import annotations

import numpy as np

from . import philox

SUPPORTED_BITS = (1, 2, 4, 8, 32)


def row_words(d: int, b: int) -> int:
    if b == 32:
        return d
    return (d * b + 31) // 32


def word_offsets(bits: np.ndarray, d: int) -> np.ndarray:
    sizes = np.array([row_words(d, int(b)) for b in bits], dtype=np.int64)
    off = np.zeros(bits.size + 1, dtype=np.int64)
    np.cumsum(sizes, out=off[1:])
    return off


def quantize_rows(h: np.ndarray, bits: np.ndarray, thresholds: np.ndarray):
    """Quantise each row of ``h`` (float32 [n, D]) with its width; ``thresholds`` are uint16 values.

    Returns (codes uint32 [n, D] -- raw float bits for b = 32 --, scale float32 [n], zero_point float32 [n]).
    """
    h = np.ascontiguousarray(h, dtype=np.float32)
    n, d = h.shape
    codes = np.zeros((n, d), dtype=np.uint32)
    scale = np.zeros(n, dtype=np.float32)
    zp = np.zeros(n, dtype=np.float32)
    for b in np.unique(bits):
        rows = np.flatnonzero(bits == b)
        x = h[rows]
        if b == 32:
            codes[rows] = x.view(np.uint32)
            continue
        L = np.float32(2 ** int(b) - 1)
        mn = x.min(axis=1)
        mx = x.max(axis=1)
        z = (mn + np.float32(0.0)).astype(np.float32)
        rng = (mx - mn).astype(np.float32)
        safe = np.where(rng == np.float32(0.0), np.float32(1.0), rng).astype(np.float32)
        with np.errstate(over="ignore"):
            inv = (L / safe).astype(np.float32)                               # fl(L / range)
        # zero range, or a range so small (< L / FLT_MAX) that its reciprocal overflows:
        # sent as the zero-scale boundary, every element reconstructs to min
        flat = (rng == np.float32(0.0)) | ~np.isfinite(inv)
        inv = np.where(flat, np.float32(0.0), inv).astype(np.float32)
        sc = np.where(flat, np.float32(0.0), safe / L).astype(np.float32)    # fl(range / L)
        t = (x - mn[:, None]).astype(np.float32)
        y = (t * inv[:, None]).astype(np.float32)
        f = np.floor(y)
        fr = (y - f).astype(np.float32)
        u = thresholds[rows].astype(np.float32)
        up = u < fr * np.float32(65536.0)
        q = np.minimum(f + up.astype(np.float32), L).astype(np.uint32)
        q[flat] = 0
        codes[rows] = q
        scale[rows] = sc
        zp[rows] = z
    return codes, scale, zp


def stochastic_quantize(h: np.ndarray, bits: np.ndarray, seed: int, epoch: int, stream_id: int,
                        node_ids: np.ndarray):
    """The sender's step: draws thresholds from Philox for (node, feature, epoch, stream) and quantises."""
    thr = philox.rounding_thresholds(node_ids, h.shape[1], seed, epoch, stream_id)
    return quantize_rows(h, np.asarray(bits), thr)


def pack(codes: np.ndarray, bits: np.ndarray):
    """Concatenate the packed rows.  Returns (words uint32 [total], word_offset int64 [n+1])."""
    n, d = codes.shape
    off = word_offsets(bits, d)
    words = np.zeros(int(off[-1]), dtype=np.uint32)
    for b in np.unique(bits):
        rows = np.flatnonzero(bits == b)
        if rows.size == 0:
            continue
        b = int(b)
        nw = row_words(d, b)
        if b == 32:
            blk = codes[rows]
        else:
            q = codes[rows].astype(np.uint64)
            pos = np.arange(d, dtype=np.int64) * b
            w_of = pos // 32
            sh = (pos % 32).astype(np.uint64)
            blk = np.zeros((rows.size, nw), dtype=np.uint64)
            for j in range(d):          # b divides 32, so a code never straddles two words
                blk[:, w_of[j]] |= q[:, j] << sh[j]
            blk = blk.astype(np.uint32)
        dst = off[rows][:, None] + np.arange(nw)[None, :]
        words[dst] = blk
    return words, off


def unpack(words: np.ndarray, word_offset: np.ndarray, bits: np.ndarray, d: int) -> np.ndarray:
    n = bits.size
    codes = np.zeros((n, d), dtype=np.uint32)
    for b in np.unique(bits):
        rows = np.flatnonzero(bits == b)
        b = int(b)
        nw = row_words(d, b)
        blk = words[word_offset[rows][:, None] + np.arange(nw)[None, :]]
        if b == 32:
            codes[rows] = blk
            continue
        pos = np.arange(d, dtype=np.int64) * b
        mask = np.uint32((1 << b) - 1)
        codes[rows] = (blk[:, pos // 32] >> (pos % 32).astype(np.uint32)) & mask
    return codes


def dequantize(codes: np.ndarray, scale: np.ndarray, zp: np.ndarray, bits: np.ndarray) -> np.ndarray:
    """The receiver's step: scale * q + zero_point in float32 (raw float for b = 32)."""
    out = np.empty(codes.shape, dtype=np.float32)
    raw = bits == 32
    out[raw] = codes[raw].view(np.float32)
    q = codes[~raw].astype(np.float32)
    out[~raw] = ((scale[~raw, None] * q).astype(np.float32) + zp[~raw, None]).astype(np.float32)
    return out
