"""Pins of the oracle's stochastic quantiser (SYLVIE guide, section 6 and the checklist of section 16).

Each pin fixes the result by something other than the oracle's own formula: closed forms on grid
rows, the two-valued and constant special cases, unbiasedness and the variance D*scale^2/6 measured
over thousands of independent draws, the |error| <= scale bound, and a big-integer reference for
the bit layout.
"""
import numpy as np
import pytest

from oracle import quantize as Q

BITS = (1, 2, 4, 8)


def _thr(rng, shape):
    return rng.integers(0, 65536, size=shape, dtype=np.uint32)


@pytest.mark.parametrize("b", BITS)
def test_grid_rows_are_exact_for_any_threshold(b):
    """x = mn + i*s with s a power of two and i in [0, L]: the scaled value is an integer, so
    stochastic rounding has nothing to round and q = i whatever the random draw."""
    rng = np.random.default_rng(b)
    L = 2 ** b - 1
    d = max(16, L + 1)
    for s_exp in (-6, 0, 3):
        s = np.float32(2.0 ** s_exp)
        i = rng.integers(0, L + 1, size=(40, d))
        i[:, 0], i[:, 1] = 0, L                       # the row spans the full range
        mn = np.float32(-37.0) * s
        x = (mn + i.astype(np.float32) * s).astype(np.float32)
        for _ in range(3):
            codes, scale, zp = Q.quantize_rows(x, np.full(40, b, np.uint8), _thr(rng, x.shape))
            np.testing.assert_array_equal(codes, i.astype(np.uint32))
            np.testing.assert_array_equal(scale, np.full(40, s, np.float32))
            np.testing.assert_array_equal(zp, np.full(40, mn, np.float32))
            back = Q.dequantize(codes, scale, zp, np.full(40, b, np.uint8))
            np.testing.assert_array_equal(back, x)


def test_one_bit_two_valued_rows_code_the_maximum():
    rng = np.random.default_rng(3)
    a = rng.standard_normal(200).astype(np.float32)
    c = (a + np.abs(rng.standard_normal(200)).astype(np.float32) + np.float32(1e-3)).astype(np.float32)
    pick = rng.integers(0, 2, size=(200, 32))
    pick[:, 0], pick[:, 1] = 0, 1
    x = np.where(pick == 1, c[:, None], a[:, None]).astype(np.float32)
    codes, scale, zp = Q.quantize_rows(x, np.ones(200, np.uint8), _thr(rng, x.shape))
    np.testing.assert_array_equal(codes, pick.astype(np.uint32))
    np.testing.assert_array_equal(zp, a)


@pytest.mark.parametrize("b", BITS)
def test_constant_rows_hit_the_zero_scale_boundary(b):
    vals = np.array([0.0, -0.0, 1.5, -3.25e-3, 7e20], dtype=np.float32)
    x = np.repeat(vals[:, None], 24, axis=1)
    codes, scale, zp = Q.quantize_rows(x, np.full(5, b, np.uint8), np.full(x.shape, 123, np.uint32))
    assert not codes.any()
    assert not scale.any()
    # min is sent as the zero-point; -0 is canonicalised to +0
    np.testing.assert_array_equal(zp.view(np.uint32), (vals + np.float32(0)).view(np.uint32))
    assert zp.view(np.uint32)[1] == 0
    back = Q.dequantize(codes, scale, zp, np.full(5, b, np.uint8))
    np.testing.assert_array_equal(back, x + np.float32(0))


def test_reciprocal_overflow_is_treated_as_zero_range():
    x = np.zeros((2, 16), np.float32)
    x[0, 3] = np.float32(1e-40)            # subnormal range: 255 / range overflows
    x[1, 3] = np.float32(1e-30)            # normal tiny range: finite reciprocal
    codes, scale, zp = Q.quantize_rows(x, np.array([8, 8], np.uint8), np.zeros(x.shape, np.uint32))
    assert scale[0] == 0 and not codes[0].any()
    assert scale[1] > 0 and codes[1, 3] == 255


def test_raw_passthrough_at_32_bits():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((10, 16)).astype(np.float32)
    x[0, 0] = -0.0
    codes, scale, zp = Q.quantize_rows(x, np.full(10, 32, np.uint8), _thr(rng, x.shape))
    np.testing.assert_array_equal(codes, x.view(np.uint32))
    assert not scale.any() and not zp.any()
    np.testing.assert_array_equal(Q.dequantize(codes, scale, zp, np.full(10, 32, np.uint8)).view(np.uint32),
                                  x.view(np.uint32))


@pytest.mark.parametrize("b", BITS)
def test_code_range_min_and_error_bound(b):
    rng = np.random.default_rng(10 + b)
    x = (rng.standard_normal((500, 64)) * rng.uniform(1e-3, 1e3, size=(500, 1))).astype(np.float32)
    bits = np.full(500, b, np.uint8)
    codes, scale, zp = Q.quantize_rows(x, bits, _thr(rng, x.shape))
    L = 2 ** b - 1
    assert codes.max() <= L
    # the minimum element has a zero fractional part and always codes to 0
    amin = x.argmin(axis=1)
    assert not codes[np.arange(500), amin].any()
    back = Q.dequantize(codes, scale, zp, bits).astype(np.float64)
    err = np.abs(back - x.astype(np.float64))
    ulp = np.spacing(np.abs(x).max(axis=1)).astype(np.float64)
    assert (err <= scale[:, None] * (1 + 1e-5) + 4 * ulp[:, None]).all()


@pytest.mark.parametrize("b", BITS)
def test_unbiased_over_independent_draws(b):
    """E[Deq(Q(h))] = h: the mean reconstruction over S draws approaches the input."""
    S = 4096
    rng = np.random.default_rng(20 + b)
    h = rng.standard_normal((1, 32)).astype(np.float32)
    bits = np.array([b], np.uint8)
    acc = np.zeros(32)
    node = np.array([5], dtype=np.uint64)
    for e in range(S):
        codes, scale, zp = Q.stochastic_quantize(h, bits, seed=0xABCDEF, epoch=e, stream_id=0, node_ids=node)
        acc += Q.dequantize(codes, scale, zp, bits)[0]
    mean_err = acc / S - h[0].astype(np.float64)
    s = float(scale[0])
    # per element: sd of one draw <= scale/2; bias of the 16-bit rule < 2^-16 scale
    assert (np.abs(mean_err) <= 5 * s / (2 * np.sqrt(S)) + s * 2.0 ** -16).all(), np.abs(mean_err).max() / s
    # pooled over the 32 elements the mean error is tighter still
    assert abs(mean_err.mean()) <= 5 * s / (2 * np.sqrt(S * 32)) + s * 2.0 ** -16


def test_variance_is_d_scale_squared_over_six():
    """Var(h~) = D*scale^2/6 when fractional parts are spread uniformly over (0, 1)."""
    S, D = 3000, 256
    s = np.float32(2.0 ** -4)
    mn = np.float32(-8.0)
    k = np.arange(D) % 255
    frac = (np.arange(D) + 0.5) / D
    y = k + frac
    y[0], y[-1] = 0.0, 255.0                            # pin min and max on the grid
    x = (mn + (y * s)).astype(np.float32)[None, :]
    assert np.array_equal(((x.astype(np.float64) - mn) / s)[0], y)
    bits = np.array([8], np.uint8)
    samples = np.empty((S, D))
    for e in range(S):
        codes, scale, zp = Q.stochastic_quantize(x, bits, seed=77, epoch=e, stream_id=1,
                                                 node_ids=np.array([9], np.uint64))
        assert scale[0] == s
        samples[e] = Q.dequantize(codes, scale, zp, bits)[0]
    total_var = samples.var(axis=0).sum()
    expect = D * float(s) ** 2 / 6
    assert abs(total_var / expect - 1) < 0.05, total_var / expect
    # and element-wise it follows scale^2 * f (1 - f)
    fr = y - np.floor(y)
    np.testing.assert_allclose(samples.var(axis=0), float(s) ** 2 * fr * (1 - fr), atol=float(s) ** 2 * 0.04)


def test_round_up_probability_equals_fraction():
    """Over all 2^16 thresholds the fraction that round up is ceil(fr * 2^16) / 2^16."""
    u = np.arange(65536, dtype=np.uint32)
    for fr_num in (1, 1000, 32768, 50000, 65535):
        y = np.float32(3 + fr_num / 65536.0)
        x = np.array([[0.0, float(y) * 0.25, 255 * 0.25]], np.float32)   # scale 0.25 at b=8
        xs = np.repeat(x, 65536, axis=0)
        thr = np.zeros(xs.shape, np.uint32)
        thr[:, 1] = u
        codes, scale, zp = Q.quantize_rows(xs, np.full(65536, 8, np.uint8), thr)
        assert scale[0] == np.float32(0.25)
        ups = int((codes[:, 1] == 4).sum())
        assert ups == fr_num


@pytest.mark.parametrize("b", BITS + (32,))
@pytest.mark.parametrize("d", (16, 48, 128))
def test_packing_against_big_integer_layout(b, d):
    rng = np.random.default_rng(b * 1000 + d)
    n = 9
    if b == 32:
        codes = rng.integers(0, 2**32, size=(n, d), dtype=np.uint64).astype(np.uint32)
    else:
        codes = rng.integers(0, 2**b, size=(n, d), dtype=np.uint32)
    bits = np.full(n, b, np.uint8)
    words, off = Q.pack(codes, bits)
    nw = d if b == 32 else -(-d * b // 32)
    assert off[-1] == n * nw
    for r in range(n):
        big = 0
        step = 32 if b == 32 else b
        for j in range(d):
            big |= int(codes[r, j]) << (j * step)
        expect = [(big >> (32 * w)) & 0xFFFFFFFF for w in range(nw)]
        assert list(words[off[r]:off[r + 1]]) == expect
    np.testing.assert_array_equal(Q.unpack(words, off, bits, d), codes)


def test_mixed_width_rows_are_laid_out_in_caller_order():
    rng = np.random.default_rng(1)
    bits = np.array([8, 1, 32, 2, 4, 1], np.uint8)
    d = 16
    codes = np.stack([rng.integers(0, 2 ** min(int(b), 31), size=d, dtype=np.uint64) for b in bits]).astype(np.uint32)
    words, off = Q.pack(codes, bits)
    np.testing.assert_array_equal(off, [0, 4, 5, 21, 22, 24, 25])
    np.testing.assert_array_equal(Q.unpack(words, off, bits, d), codes)
