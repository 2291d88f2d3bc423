"""Pins for the oracle's dynamic-tree codebooks (CPU only).

What the summary page fixes (§2 "Dynamic Quantization", §2 "Block-wise
Quantization"): the bit layout (sign, a run of zeros as exponent, an indicator bit,
a linear fraction), the unsigned variant that reuses the sign bit for the fraction,
and the normalised range [-1, 1].  The tests below check those facts and the
arithmetic of the binary32 rounding with methods independent of the oracle's code.
"""

from fractions import Fraction
import json
import os

import numpy as np
import pytest

import oracle
from oracle import SIGNED, UNSIGNED

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _from_bit_string(bits):
    """Decode a magnitude bit string by reading characters: zeros, indicator, fraction."""
    e = 0
    while e < len(bits) and bits[e] == "0":
        e += 1
    if e == len(bits):
        return Fraction(0)
    assert bits[e] == "1"            # the indicator bit
    frac_bits = bits[e + 1:]
    f = len(frac_bits)
    j = int(frac_bits, 2) if f else 0
    # linear fraction over 2^f steps of the decade [0.1, 1], right end points
    step = Fraction(9, 10) / (2 ** f)
    return (Fraction(1, 10) + step * (j + 1)) * Fraction(1, 10 ** e)


@pytest.mark.parametrize("kind,nb", [(SIGNED, 7), (UNSIGNED, 8)])
def test_layout_matches_bit_string_reading(kind, nb):
    exact = oracle.magnitude_rationals(kind)
    assert len(exact) == 2 ** nb
    for pattern in range(2 ** nb):
        assert exact[pattern] == _from_bit_string(format(pattern, f"0{nb}b")), pattern


@pytest.mark.parametrize("kind,nb", [(SIGNED, 7), (UNSIGNED, 8)])
def test_decades_tile_unit_interval(kind, nb):
    """Each decade (10^-(e+1), 10^-e] holds 2^(nb-1-e) equally spaced entries whose
    top is 10^-e; consecutive decades meet with no gap; the largest is exactly 1."""
    exact = oracle.magnitude_rationals(kind)[1:]
    assert max(exact) == 1
    for e in range(nb):
        dec = [q for q in exact if Fraction(1, 10 ** (e + 1)) < q <= Fraction(1, 10 ** e)]
        assert len(dec) == 2 ** (nb - 1 - e)
        assert dec[-1] == Fraction(1, 10 ** e)
        grid = [dec[0] - Fraction(1, 10 ** (e + 1))] + \
               [b - a for a, b in zip(dec, dec[1:])]
        assert len(set(grid)) == 1, f"decade {e} is not a linear grid"
    assert sum(1 for q in exact if q > 0) == 2 ** nb - 1


@pytest.mark.parametrize("kind", [SIGNED, UNSIGNED])
def test_pattern_order_is_value_order(kind):
    exact = oracle.magnitude_rationals(kind)
    assert all(a < b for a, b in zip(exact, exact[1:]))
    m = oracle.magnitudes_f32(kind)
    assert np.all(np.diff(m) > 0)
    assert m[0] == 0 and m[-1] == np.float32(1.0)


def test_extreme_entries():
    m7 = oracle.magnitudes_f32(SIGNED)
    m8 = oracle.magnitudes_f32(UNSIGNED)
    assert m7.size == 128 and m8.size == 256
    assert m7[1] == np.float32(1e-6) and m8[1] == np.float32(1e-7)
    assert m7[126] == np.float32(0.9859375)
    assert m8[254] == np.float32(0.99296875)


def _ulp32(x):
    x = np.float32(x)
    return float(np.nextafter(x, np.float32(np.inf)) - x)


@pytest.mark.parametrize("kind", [SIGNED, UNSIGNED])
def test_entries_are_correctly_rounded(kind):
    """|fp32 entry - exact rational| <= half an ulp, and no neighbour is nearer."""
    exact = oracle.magnitude_rationals(kind)
    m = oracle.magnitudes_f32(kind)
    for q, v in zip(exact, m):
        err = abs(Fraction(float(v)) - q)
        below = Fraction(float(np.nextafter(v, np.float32(-1))))
        above = Fraction(float(np.nextafter(v, np.float32(2))))
        assert err <= abs(below - q) and err <= abs(above - q)


def test_round_rational_ties_and_random():
    r = oracle.round_rational_to_f32
    one = Fraction(1)
    u = Fraction(1, 2 ** 23)
    assert r(one + u / 2) == np.float32(1.0)                          # tie -> even
    assert r(one + 3 * u / 2) == np.float32(1.0 + 2.0 ** -22)         # tie -> even
    assert r(one + u / 2 + Fraction(1, 2 ** 60)) == np.float32(1.0 + 2.0 ** -23)
    assert r(Fraction(1, 2 ** 149)) == np.float32(2.0 ** -149)        # subnormal
    assert r(Fraction(3, 2 ** 151)) == np.float32(2.0 ** -149)        # 0.75 q -> 1 q
    rng = np.random.default_rng(11)
    for _ in range(2000):
        q = Fraction(int(rng.integers(1, 2 ** 40)), int(rng.integers(1, 2 ** 40)))
        x64 = float(q)
        # skip the rare cases where binary64 lands within 2 ulps of a binary32 tie
        hi = np.float32(x64)
        mid_dist = abs(abs(x64 - float(hi)) - _ulp32(hi) / 2)
        if mid_dist < 4 * np.spacing(x64):
            continue
        assert r(q) == hi


@pytest.mark.parametrize("kind", [SIGNED, UNSIGNED])
def test_decode_table(kind):
    t = oracle.decode_table(kind)
    m = oracle.magnitudes_f32(kind)
    assert t.size == 256 and t.dtype == np.float32
    if kind == UNSIGNED:
        assert np.array_equal(t, m)
        assert t.min() == 0 and t.max() == 1
    else:
        assert np.array_equal(t[:128], m)
        assert np.array_equal(t[128:], -m)
        assert np.signbit(t[0x80]) and t[0x80] == 0
        assert t.min() == -1 and t.max() == 1     # normalised range [-1, 1]


def test_golden_tables_unchanged():
    """The committed golden tables (written by tests/golden/make_codebooks.py, which
    calls only the oracle) still match: guards against silent oracle edits."""
    for kind, name in [(SIGNED, "codebook_signed.txt"), (UNSIGNED, "codebook_unsigned.txt")]:
        rows = [ln.split() for ln in open(os.path.join(GOLDEN, name))
                if ln.strip() and not ln.startswith("#")]
        bits = np.array([int(r[1], 16) for r in rows], dtype=np.uint32)
        assert np.array_equal(bits, oracle.decode_table(kind).view(np.uint32))


def test_page_facts_fixture():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    assert facts["block_size"]["value"] == oracle.BLOCK
    lo, hi = facts["normalised_range"]["value"]
    for kind in (SIGNED, UNSIGNED):
        t = oracle.decode_table(kind)
        assert t.min() >= lo and t.max() <= hi
