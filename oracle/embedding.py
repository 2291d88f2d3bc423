"""Oracle: the Stable Embedding layer (test infrastructure only).

Sources:
* 8-bit optimizers summary page (wiki.neutronadmin.com/news/16836), §2 "Stable
  Embedding Layer": the embedding weight is initialised with Xavier uniform, and a
  layer normalisation follows the embedding lookup, so the output has variance of
  about 1; a uniform rather than normal initialisation has no extreme values.
* YaLM-100B training page (golden-irbis.ru), "Stabilizations. LayerNorm": a
  LayerNorm placed right after the embedding; "Stabilizations. BFloat 16": every
  LayerNorm is computed in tf32 / fp32 even when weights are bf16.

Readings where the pages are silent:
* Xavier uniform is Glorot and Bengio's rule: U(-a, a) with a = sqrt(6 / (fan_in +
  fan_out)); for a [rows, dim] table the two fans are dim and rows.  a is computed
  in binary64 and rounded once to binary32; each weight is fl32(a * (2u - 1)).
* The uniform numbers come from one counter-based generator, Philox4x32-10 (Salmon,
  Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011):
  element e of the row-major table uses word e % 4 of the block with counter
  (e // 4 low word, e // 4 high word, 0, 0) and key (seed low word, seed high word);
  u = (word >> 8) * 2^-24, which lies in [0, 1) on a 2^-24 grid.
* LayerNorm is the usual one over the last dimension: mean, biased variance,
  y = (x - mean) / sqrt(var + eps) * gamma + beta, with eps = 1e-5 by default.
  The oracle evaluates it in binary64; the kernels compute in binary32 (the YaLM
  page's fp32) and are compared within a bound derived from their arithmetic.
* The backward pass is the exact gradient of that forward pass: for gamma and beta
  summed over tokens, for the table scattered back to each token's row (repeated
  indices add up).

Parity: Philox pinned to the generator's published known-answer values; the Xavier
bound pinned to torch.nn.init's own rule on the same shape and to the moments of
the uniform law; the forward pinned to torch's layer_norm in binary64 and to its
invariants; the backward pinned to central finite differences of the forward and
to torch autograd in binary64.
"""

import math

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
PHILOX_ROUNDS = 10
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds.  ctr: (..., 4) uint32, key: (..., 2) uint32;
    returns (..., 4) uint32.  Each round multiplies words 0 and 2 by the two
    constants (64-bit products), and the new words are (hi(M1 c2) ^ c1 ^ k0,
    lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key is bumped by the two Weyl
    constants between rounds.  Parity: pinned (published known-answer values)."""
    c = np.asarray(ctr, dtype=np.uint32).astype(np.uint64)
    k = np.asarray(key, dtype=np.uint32).astype(np.uint64)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    for r in range(PHILOX_ROUNDS):
        if r:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = np.uint64(PHILOX_M0) * c0
        p1 = np.uint64(PHILOX_M1) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _MASK32,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _MASK32)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def uniform01(words):
    """[0, 1) binary32 from 32-bit words: the top 24 bits times 2^-24 (exact)."""
    w = np.asarray(words, dtype=np.uint32)
    return ((w >> np.uint32(8)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def xavier_bound(rows, dim):
    """a = sqrt(6 / (fan_in + fan_out)) rounded once to binary32.
    Parity: pinned (torch.nn.init's rule on the same shape)."""
    return np.float32(math.sqrt(6.0 / float(int(rows) + int(dim))))


def xavier_uniform(rows, dim, seed):
    """The [rows, dim] binary32 table of the initialisation above.
    Parity: pinned through philox4x32_10 and xavier_bound, plus the moments of
    the uniform law."""
    n = int(rows) * int(dim)
    e = np.arange(n, dtype=np.uint64)
    blk = e // np.uint64(4)
    ctr = np.zeros((n, 4), dtype=np.uint32)
    ctr[:, 0] = (blk & _MASK32).astype(np.uint32)
    ctr[:, 1] = (blk >> np.uint64(32)).astype(np.uint32)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32)
    words = philox4x32_10(ctr, np.broadcast_to(key, (n, 2)))
    u = uniform01(words[np.arange(n), (e % np.uint64(4)).astype(np.int64)])
    a = xavier_bound(rows, dim)
    two_u_minus_1 = (np.float32(2.0) * u) - np.float32(1.0)   # exact in binary32
    return (a * two_u_minus_1).astype(np.float32).reshape(int(rows), int(dim))


def layer_norm_rows(x, gamma, beta, eps):
    """Row-wise LayerNorm in binary64: returns (y, mean, rstd, xhat).
    Parity: pinned (torch layer_norm in binary64, invariants)."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + float(eps))
    xhat = (x - mean) * rstd
    y = xhat * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)
    return y, mean[..., 0], rstd[..., 0], xhat


def stable_embedding_forward(weight, idx, gamma, beta, eps=1e-5):
    """y[t] = LayerNorm(weight[idx[t]]) in binary64: returns (y, mean, rstd).
    Parity: pinned (see layer_norm_rows)."""
    w = np.asarray(weight, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size and (idx.min() < 0 or idx.max() >= w.shape[0]):
        raise IndexError("index out of range")
    y, mean, rstd, _ = layer_norm_rows(w[idx], gamma, beta, eps)
    return y, mean, rstd


def stable_embedding_backward(weight, idx, gamma, beta, dy, eps=1e-5):
    """Gradients of sum(y * dy) for the forward above, in binary64:
    returns (dweight [rows, dim], dgamma [dim], dbeta [dim]).

    With xhat = (x - mean) * rstd and g = dy * gamma:
      dx = rstd * (g - mean(g) - xhat * mean(g * xhat))   (row means over dim)
      dgamma = sum over tokens of dy * xhat, dbeta = sum over tokens of dy,
      dweight[r] = sum of dx over the tokens t with idx[t] = r.
    Parity: pinned (central finite differences, torch autograd in binary64)."""
    w = np.asarray(weight, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    dy = np.asarray(dy, dtype=np.float64)
    _, _, rstd, xhat = layer_norm_rows(w[idx], gamma, beta, eps)
    g = dy * np.asarray(gamma, np.float64)
    c1 = g.mean(axis=-1, keepdims=True)
    c2 = (g * xhat).mean(axis=-1, keepdims=True)
    dx = rstd[:, None] * (g - c1 - xhat * c2)
    dweight = np.zeros_like(w)
    np.add.at(dweight, idx, dx)
    return dweight, (dy * xhat).sum(axis=0), dy.sum(axis=0)
