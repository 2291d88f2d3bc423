"""Oracle: the dynamic-tree codebooks (test infrastructure only).

Source: 8-bit optimizers summary page, §2 "Dynamic Quantization".  A dynamic-tree
code is read from its most significant bit: a sign bit, then a run of zero bits
whose length is the exponent, then an indicator bit (1) announcing that the
remaining bits are a linear fraction.  The unsigned variant drops the sign bit
and gives that bit to the fraction.  §2 "Block-wise Quantization" fixes the value
range of the normalised codes to [-1, 1].

Readings where the page is silent (parity against the page itself is unpinned on
these points, because the page prints no code values):

* Exponent base 10: a run of e zeros scales by 10^-e.  (The page does not name a
  base; base 10 is the reading that gives the 1e-6 / 1e-7 dynamic range an
  optimizer state needs, while base 2 would stop at 2^-7.)
* The f fraction bits with integer value j place the magnitude on the right end
  of the j-th of 2^f equal sub-intervals of [0.1, 1]:
  ``10^-e * (0.1 + 0.9 * (j + 1) / 2^f)``.  So each decade (0.1, 1] * 10^-e is
  tiled with no gap, and 1.0 itself is a code.
* The all-zero magnitude pattern is the value 0.
* Signed codes are sign-magnitude: byte = sign << 7 | magnitude pattern, so the
  byte 0x80 decodes to -0.0.
* The stored table value is the binary32 nearest to the exact rational (ties to
  even), i.e. the plain correctly rounded value.
"""

from fractions import Fraction
import functools
import math

import numpy as np

BLOCK = 2048  # §2 "Block-wise Quantization": blocks of 2048 elements
SIGNED = 0
UNSIGNED = 1

# number of magnitude bits: the signed code spends one of its 8 bits on the sign
_MAG_BITS = {SIGNED: 7, UNSIGNED: 8}


def magnitude_rationals(kind):
    """Exact magnitudes of every magnitude bit pattern, in pattern order.

    Entry P is the magnitude encoded by the bit pattern P (P = 0 .. 2^nb - 1), with
    nb = 7 magnitude bits for the signed code and 8 for the unsigned one.  Pattern
    P > 0 is decoded literally from its bits, most significant first: count the
    leading zero bits (exponent e), skip the indicator 1 bit, and read the f
    remaining bits as the fraction integer j.  Parity: pinned (independent
    bit-string construction, tiling and ordering invariants in
    tests/test_oracle_codebook.py).
    """
    nb = _MAG_BITS[kind]
    out = [Fraction(0)]
    for pattern in range(1, 1 << nb):
        indicator_pos = pattern.bit_length() - 1  # index of the leading 1 bit
        e = nb - 1 - indicator_pos                # zero bits above the indicator
        f = indicator_pos                         # fraction bits below it
        j = pattern - (1 << f)
        frac = Fraction(1, 10) + Fraction(9, 10) * Fraction(j + 1, 1 << f)
        out.append(frac / (10 ** e))
    return out


def round_rational_to_f32(q):
    """Binary32 value nearest to the non-negative rational q, ties to even.

    Plain definition of IEEE round-to-nearest-even, done in exact integer
    arithmetic (subnormal results use the fixed quantum 2^-149).  Parity: pinned
    against numpy's float64 -> float32 conversion where no double rounding can
    occur and against the half-ulp bound.
    """
    q = Fraction(q)
    if q < 0:
        raise ValueError("negative rational")
    if q == 0:
        return np.float32(0.0)
    n, d = q.numerator, q.denominator
    # exponent E with 2^E <= q < 2^(E+1)
    E = n.bit_length() - d.bit_length()
    if _cmp_pow2(n, d, E) < 0:
        E -= 1
    E = max(E, -126)
    shift = E - 23  # value of the last mantissa bit
    scaled = q / (Fraction(2) ** shift)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and (m & 1)):
        m += 1
    val = math.ldexp(float(m), shift)  # m < 2^25, exact in binary64
    if val > float(np.finfo(np.float32).max):
        raise OverflowError("rational beyond binary32 range")
    return np.float32(val)


def _cmp_pow2(n, d, E):
    """Sign of n/d - 2^E, exactly."""
    if E >= 0:
        lhs, rhs = n, d << E
    else:
        lhs, rhs = n << (-E), d
    return (lhs > rhs) - (lhs < rhs)


@functools.lru_cache(maxsize=None)
def _magnitudes_f32_cached(kind):
    t = np.array([round_rational_to_f32(q) for q in magnitude_rationals(kind)],
                 dtype=np.float32)
    t.setflags(write=False)
    return t


def magnitudes_f32(kind):
    """Binary32 magnitude table, index = magnitude pattern (ascending values)."""
    return _magnitudes_f32_cached(kind)


def decode_table(kind):
    """256-entry decode table indexed by the stored code byte.

    Unsigned: byte = magnitude pattern.  Signed: bit 7 is the sign, bits 0..6 the
    magnitude pattern; a set sign bit negates (so 0x80 gives -0.0).
    """
    return _decode_table_cached(kind)


@functools.lru_cache(maxsize=None)
def _decode_table_cached(kind):
    mags = magnitudes_f32(kind)
    if kind == UNSIGNED:
        out = mags.copy()
    else:
        out = np.empty(256, dtype=np.float32)
        for byte in range(256):
            mag = mags[byte & 0x7F]
            out[byte] = -mag if (byte & 0x80) else mag
    out.setflags(write=False)
    return out
