"""Pins for the oracle's block-wise quantize / dequantize (CPU only).

Facts from the summary page: blocks of 2048 normalised independently by their own
absmax, so an outlier only changes its own block (§2 "Block-wise Quantization");
quantization stores the nearest representable value and dequantization maps back
(§1).  Checks: brute force, round trips, error bounds, block independence, tails.
"""

import numpy as np
import pytest

import oracle
from oracle import SIGNED, UNSIGNED, BLOCK

KINDS = [SIGNED, UNSIGNED]


def _adversarial_points(mags):
    """Table entries, midpoints and decade edges, each +- a few ulps, plus extremes."""
    pts = [0.0, 1.0, np.float32(1.0) + np.float32(2 ** -23), 1e-30, 2.0 ** -126]
    mids = (mags[:-1].astype(np.float64) + mags[1:]) / 2
    for c in list(mags) + list(mids) + [10.0 ** -e for e in range(9)]:
        c = np.float32(c)
        pts.append(c)
        lo = hi = c
        for _ in range(4):
            lo = np.nextafter(lo, np.float32(-1))
            hi = np.nextafter(hi, np.float32(2))
            pts += [lo, hi]
    a = np.array(pts, dtype=np.float32)
    return a[a >= 0]


@pytest.mark.parametrize("kind", KINDS)
def test_nearest_matches_bruteforce(kind):
    mags = oracle.magnitudes_f32(kind)
    rng = np.random.default_rng(5)
    a = np.concatenate([
        _adversarial_points(mags),
        rng.random(3000).astype(np.float32),
        (10.0 ** rng.uniform(-8, 0, 3000)).astype(np.float32),
    ])
    got = oracle.nearest_magnitude_index(mags, a)
    want = oracle.nearest_magnitude_index_bruteforce(mags, a)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kind", KINDS)
def test_nearest_is_monotone_and_transitions_consistent(kind):
    """The rule is a non-decreasing step function of a; each transition point T[k]
    maps to k and its predecessor to k - 1 (checked on a strided sweep of the
    binary32s in [0, 1.01], every 1009th, and densely around each transition)."""
    mags = oracle.magnitudes_f32(kind)
    hi_bits = int(np.float32(1.01).view(np.uint32))
    bits = np.arange(0, hi_bits, 1009, dtype=np.uint32)
    a = bits.view(np.float32)
    idx = oracle.nearest_magnitude_index(mags, a)
    assert np.all(np.diff(idx) >= 0)
    T = oracle.code_transitions(kind)
    assert T.size == mags.size - 1 and np.all(np.diff(T) > 0)
    k = np.arange(1, mags.size)
    assert np.array_equal(oracle.nearest_magnitude_index(mags, T), k)
    prev = np.nextafter(T, np.float32(-1))
    assert np.array_equal(oracle.nearest_magnitude_index(mags, prev), k - 1)
    # dense +-256 ulps around every transition, compared with the step function
    tb = T.view(np.uint32).astype(np.int64)
    around = (tb[:, None] + np.arange(-256, 257)[None, :]).reshape(-1)
    around = around[around >= 0].astype(np.uint32).view(np.float32)
    want = np.searchsorted(T, around, side="right")
    assert np.array_equal(oracle.nearest_magnitude_index(mags, around), want)
    # and the strided sweep agrees with the step function too
    assert np.array_equal(idx, np.searchsorted(T, a, side="right"))


@pytest.mark.parametrize("kind", KINDS)
def test_round_trip_of_table_values(kind):
    """Blocks made of table values times a scale, with one element equal to the
    scale, quantize back to the same codes (0x80 decodes to -0 and re-encodes to
    0x00, its value-equal code)."""
    table = oracle.decode_table(kind)
    rng = np.random.default_rng(7)
    for scale in [np.float32(1.0), np.float32(2.0 ** -10), np.float32(3.7e-3),
                  np.float32(rng.normal() ** 2 + 0.5)]:
        codes = rng.integers(0, 256, BLOCK).astype(np.uint8)
        codes[17] = 0x7F if kind == SIGNED else 0xFF        # an element at +scale
        x = table[codes] * scale
        c2, am = oracle.quantize_blockwise(x, kind)
        assert am[0] == scale
        want = codes.copy()
        if kind == SIGNED:
            want[want == 0x80] = 0x00
        assert np.array_equal(c2, want)
        y = oracle.dequantize_blockwise(c2, am, kind)
        assert np.array_equal(np.abs(y), np.abs(x))


@pytest.mark.parametrize("kind", KINDS)
def test_dequantization_error_bound(kind):
    """|x - deq(q(x))| <= absmax * (half the local table gap) plus binary32 slop."""
    mags = oracle.magnitudes_f32(kind).astype(np.float64)
    rng = np.random.default_rng(3)
    x = (0.01 * rng.standard_t(3, 5 * BLOCK + 77)).astype(np.float32)
    if kind == UNSIGNED:
        x = np.abs(x)
    c, am = oracle.quantize_blockwise(x, kind)
    y = oracle.dequantize_blockwise(c, am, kind)
    A = np.repeat(am, BLOCK)[: x.size].astype(np.float64)
    a = np.abs(x.astype(np.float64)) / A
    lo = np.clip(np.searchsorted(mags, a, side="right") - 1, 0, mags.size - 2)
    gap = mags[lo + 1] - mags[lo]
    bound = A * (0.5 * gap) * (1 + 1e-6) + 4 * np.finfo(np.float32).eps * A
    assert np.all(np.abs(x.astype(np.float64) - y) <= bound)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("factor", [100.0, 1000.0])
def test_outlier_changes_only_its_block(kind, factor):
    rng = np.random.default_rng(9)
    n = 7 * BLOCK + 300
    x = rng.normal(0, 1e-3, n).astype(np.float32)
    if kind == UNSIGNED:
        x = np.abs(x)
    c0, a0 = oracle.quantize_blockwise(x, kind)
    for pos in [5, 3 * BLOCK + 1000, n - 1]:
        x2 = x.copy()
        x2[pos] *= np.float32(factor)
        c1, a1 = oracle.quantize_blockwise(x2, kind)
        b = pos // BLOCK
        s, e = b * BLOCK, min(n, (b + 1) * BLOCK)
        assert a1[b] != a0[b]
        keep = np.ones(n, bool)
        keep[s:e] = False
        assert np.array_equal(c1[keep], c0[keep])
        assert np.array_equal(np.delete(a1, b), np.delete(a0, b))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n", [1, 7, 2047, 2048, 2049, 50257, 3 * 2048 + 5])
def test_tails_are_own_blocks(kind, n):
    """The last short block only sees its own elements: quantizing it alone gives
    the same codes and absmax."""
    rng = np.random.default_rng(n)
    x = rng.normal(0, 1, n).astype(np.float32)
    c, a = oracle.quantize_blockwise(x, kind)
    assert c.size == n and a.size == -(-n // BLOCK)
    s = (a.size - 1) * BLOCK
    c_t, a_t = oracle.quantize_blockwise(x[s:], kind)
    assert np.array_equal(c[s:], c_t) and a[-1] == a_t[0]
    assert a[-1] == np.abs(x[s:]).max()


@pytest.mark.parametrize("kind", KINDS)
def test_zero_and_subnormal_blocks(kind):
    x = np.zeros(3 * BLOCK, np.float32)
    x[BLOCK:2 * BLOCK] = np.float32(1e-40)          # subnormal block
    x[2 * BLOCK + 3] = np.float32(-0.5 if kind == SIGNED else 0.5)
    c, a = oracle.quantize_blockwise(x, kind)
    assert a[0] == 0 and a[1] == 0 and a[2] == np.float32(0.5)
    assert not c[: 2 * BLOCK].any()
    y = oracle.dequantize_blockwise(np.zeros(5, np.uint8), np.zeros(1, np.float32), kind)
    assert np.array_equal(y, np.zeros(5, np.float32))


def test_signs_and_negative_zero():
    x = np.array([-0.0, 0.0, -1.0, 1.0, -1e-9, 1e-9], np.float32)
    c, a = oracle.quantize_blockwise(x, SIGNED)
    assert a[0] == 1.0
    assert list(c) == [0x00, 0x00, 0xFF, 0x7F, 0x80, 0x00]
    cu, au = oracle.quantize_blockwise(x, UNSIGNED)
    cu2, _ = oracle.quantize_blockwise(np.abs(x), UNSIGNED)
    assert np.array_equal(cu, cu2)   # unsigned codes encode |x|
