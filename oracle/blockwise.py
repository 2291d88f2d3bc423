"""Oracle: block-wise quantization and dequantization (test infrastructure only).

Source: 8-bit optimizers summary page.
* §2 "Block-wise Quantization": the tensor is cut into blocks of 2048 elements;
  each block is normalised into [-1, 1] by its own absolute maximum, computed
  independently of every other block, so an outlier only affects its own block.
* §1: quantization represents fp32 values with fewer bits after normalising them
  into a range; dequantization maps the stored values back.
* §2 "Dynamic Quantization": the codebooks (see codebook.py).

Readings where the page is silent:
* Blocks are counted from element 0 of each tensor; the last block may be short
  and uses only its own elements.
* Normalisation multiplies by one per-block reciprocal r = fl32(1 / absmax)
  instead of dividing every element (the same in exact arithmetic).
* The code of a normalised magnitude a is the nearest table magnitude, distances
  measured in binary32 (fl32(M[k+1] - a) against fl32(a - M[k])); an exact tie
  goes to the smaller magnitude.
* Signed codes put x < 0 in bit 7 (so -0.0 gives 0x00, and a negative value whose
  magnitude rounds to zero gives 0x80).  Unsigned codes encode |x|.
* A block whose absmax is below the smallest normal binary32 (2^-126, this covers
  an all-zero block) is stored as absmax 0 with every code 0: its reciprocal
  would overflow, and such values are far below any Adam epsilon.
* Dequantization is one binary32 multiply: value = table[code] * absmax.
"""

import numpy as np

from .codebook import BLOCK, SIGNED, UNSIGNED, magnitudes_f32, decode_table

FLT_MIN = np.float32(np.finfo(np.float32).tiny)  # 2^-126


def nearest_magnitude_index(mags, a):
    """Index of the table magnitude nearest to each a >= 0 (ties to the lower one).

    lo is the largest index with mags[lo] <= a (mags[0] = 0 <= a always); the code
    moves up to lo + 1 only when that neighbour is strictly nearer in binary32.
    Parity: pinned against brute force and the transition structure.
    """
    mags = np.asarray(mags, dtype=np.float32)
    a = np.asarray(a, dtype=np.float32)
    last = mags.size - 1
    lo = np.searchsorted(mags, a, side="right") - 1
    hi = np.minimum(lo + 1, last)
    up = mags[hi] - a          # binary32 subtraction
    down = a - mags[lo]
    go_up = (lo < last) & (up < down)
    return np.where(go_up, lo + 1, lo).astype(np.int64)


def nearest_magnitude_index_bruteforce(mags, a):
    """argmin_k fl32(|a - mags[k]|), lowest k on ties: for pinning only."""
    mags = np.asarray(mags, dtype=np.float32)
    a = np.asarray(a, dtype=np.float32).reshape(-1)
    out = np.empty(a.size, dtype=np.int64)
    for i, ai in enumerate(a):
        dist = np.abs(ai - mags)          # binary32 per entry
        out[i] = int(np.argmin(dist))     # argmin returns the first minimum
    return out


def _block_slices(n):
    for start in range(0, n, BLOCK):
        yield start, min(start + BLOCK, n)


def quantize_blockwise(x, kind):
    """Quantize a 1-D fp32 array into (codes uint8[n], absmax fp32[ceil(n/2048)]).

    Parity: pinned (round trip of table values, brute-force nearest code, error
    bound, block independence, zero and tail handling).
    """
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    n = x.size
    nblocks = -(-n // BLOCK)
    mags = magnitudes_f32(kind)
    codes = np.zeros(n, dtype=np.uint8)
    absmax = np.zeros(nblocks, dtype=np.float32)
    for b, (s, e) in enumerate(_block_slices(n)):
        blk = x[s:e]
        mag = np.abs(blk)
        A = mag.max()
        if not A >= FLT_MIN:
            continue  # zero or subnormal block: absmax 0, codes 0
        r = np.float32(1.0) / A
        a = mag * r
        k = nearest_magnitude_index(mags, a)
        if kind == SIGNED:
            k = np.where(blk < 0, k | 0x80, k)
        codes[s:e] = k.astype(np.uint8)
        absmax[b] = A
    return codes, absmax


def dequantize_blockwise(codes, absmax, kind):
    """Inverse map: fp32 value = decode_table[code] * absmax of the element's block."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    absmax = np.asarray(absmax, dtype=np.float32).reshape(-1)
    n = codes.size
    if absmax.size != -(-n // BLOCK):
        raise ValueError("absmax must hold ceil(n / 2048) entries")
    table = decode_table(kind)
    out = np.empty(n, dtype=np.float32)
    for b, (s, e) in enumerate(_block_slices(n)):
        out[s:e] = table[codes[s:e]] * absmax[b]
    return out


def code_transitions(kind):
    """Smallest binary32 a >= 0 at which the nearest index becomes k, k = 1..last.

    Found by bisection over binary32 bit patterns (monotone for a >= 0), using only
    ``nearest_magnitude_index``.  Valid because the nearest-index rule is a
    non-decreasing step function of a (checked by tests on dense sweeps).  Used to
    state the expected codes of an ordered sweep of every binary32 in [0, 1].
    """
    mags = magnitudes_f32(kind)
    last = mags.size - 1
    out = np.empty(last, dtype=np.float32)
    lo_bits = np.zeros(last, dtype=np.int64)                      # a = 0 -> index 0
    hi_bits = np.full(last, int(np.float32(1.0).view(np.uint32)), dtype=np.int64)
    ks = np.arange(1, last + 1)
    # invariant: index(lo) < k <= index(hi)
    while True:
        active = hi_bits - lo_bits > 1
        if not active.any():
            break
        mid = (lo_bits + hi_bits) // 2
        idx = nearest_magnitude_index(mags, mid.astype(np.uint32).view(np.float32))
        up = idx >= ks
        hi_bits = np.where(active & up, mid, hi_bits)
        lo_bits = np.where(active & ~up, mid, lo_bits)
    out[:] = hi_bits.astype(np.uint32).view(np.float32)
    return out
