"""Error bounds for the Stable Embedding kernels against the binary64 oracle (test
helpers, shared by the GPU parity tests and the CPU tests that pin the bounds).

The kernels compute in binary32 with u = 2^-24.  k is the depth of their row sums:
per-lane sums over at most max(4 S, ceil(dim / 64)) terms, then 6 levels of additions
across the wave.  With that, the row mean is within (k + 1) u mean|x| of the exact
one, rstd within (k / 2 + 7) u relative, and so on through each operation; every
bound below is that first-order bound times 2.

The table gradient of a row r used by c tokens is the LayerNorm backward map L_r
(linear, fixed by the row's x, mean and rstd) applied to the sum of the tokens'
upstream rows:  dweight[r] = base + L_r(S_r),  S_r = sum of dy_t over those tokens.

* Grouped path (vector widths): the kernels sum the c upstream rows in binary32 and
  apply L_r once.  They sort the tokens by row and cut the sorted list into chunks of
  CHUNK tokens; within a chunk a wave adds a run's rows one after another, and a run
  that crosses chunks has its chunk partials added one after another in chunk order.
  A run touches at most ceil(c / CHUNK) + 1 chunks, so every term passes through at
  most (CHUNK - 1) + ceil(c / CHUNK) roundings (and never more than c - 1): the sum
  is within that many u times sum|dy_t| of the exact sum per element.  That error
  passes through L_r, which is bounded by its absolute map; L_r's own rounding on the
  sum is the single-token bound applied to S_r; the accumulation onto base rounds
  once.  The bound does not grow with the square of the count.  With upstream values
  on a coarse dyadic grid every binary32 partial sum is exact and the summation term
  vanishes, leaving a bound independent of c.
* Element-wise path (other widths): each token's L_r(dy_t) is formed on its own and
  scattered with float atomics: the c map errors add up, and the c + 1 term sum
  onto base is within c u (|base| + sum|L_r(dy_t)|).
"""

import numpy as np

from oracle import embedding as E

U = 2.0 ** -24
CHUNK = 32   # sorted tokens per chunk in the grouped backward kernels


def sum_depth(c, chunk=CHUNK):
    """Most roundings any term of a c-term sum passes through: chunk-wise sequential
    sums, then the chunk partials in order; c - 1 for a plain sequential sum."""
    c = np.asarray(c, np.int64)
    if chunk is None:
        return np.maximum(c - 1, 0)
    return np.minimum(np.maximum(c - 1, 0), (chunk - 1) + -(-c // chunk))


def depth(dim):
    s = 2
    while 256 * s < dim and s < 16:
        s *= 2
    per_lane = max(4 * s, -(-dim // 64)) if dim <= 4096 else -(-dim // 64)
    return per_lane + 6


def grouped_path(dim):
    """Widths whose table gradient takes the grouped path (given an aligned table)."""
    return dim % 4 == 0 and dim <= 4096


def forward_tol(x, gamma, beta, eps, out_dt):
    """Bound on |y_kernel - y_exact| per element (x: the gathered rows, binary64)."""
    k = depth(x.shape[1])
    y, mean, rstd, xhat = E.layer_norm_rows(x, gamma, beta, eps)
    mabs = np.abs(x).mean(axis=1, keepdims=True)
    tol = 2 * U * (np.abs(gamma) * ((k / 2 + 8) * np.abs(xhat) + (k + 1) * mabs * rstd[:, None])
                   + np.abs(y) + 1e-30)
    if out_dt == "bf16":
        tol = tol + 2.0 ** -8 * np.abs(y) + 2.0 ** -133
    return y, mean, rstd, tol


def map_tol(up, gamma, xh, r, mabs_x, k):
    """Rounding bound of the kernels' binary32 LayerNorm backward applied to upstream
    rows ``up`` (one row each; xh, r, mabs_x of the matching table rows)."""
    g = up * gamma
    m2 = (g * xh).mean(axis=1, keepdims=True)
    mabs_g = np.abs(g).mean(axis=1, keepdims=True)
    mabs_gx = np.abs(g * xh).mean(axis=1, keepdims=True)
    return 2 * U * (k + 16) * r * (np.abs(g) + mabs_g + np.abs(xh) * (mabs_gx + np.abs(m2))
                                   + np.abs(m2) * mabs_x * r)


def map_abs(e, gamma, xh, r):
    """Elementwise bound of |L(d)| for any d with |d| <= e (the map's absolute form)."""
    ge = np.abs(gamma) * e
    return r * (ge + ge.mean(axis=1, keepdims=True)
                + np.abs(xh) * (ge * np.abs(xh)).mean(axis=1, keepdims=True))


def row_sums(idx, dy):
    """Distinct rows of ``idx`` with, per row, the first token, the token count, the
    exact sum of the upstream rows and the sum of their magnitudes (binary64)."""
    order = np.argsort(idx, kind="stable")
    rows, starts, counts = np.unique(idx[order], return_index=True, return_counts=True)
    d = np.asarray(dy, np.float64)[order]
    S = np.add.reduceat(d, starts, axis=0)
    A = np.add.reduceat(np.abs(d), starts, axis=0)
    return rows, order[starts], counts, S, A


def dweight_tol(x_rows, idx, rows, gamma, beta, dy, eps, base=0.0, grouped=True,
                exact_sums=False):
    """Per-element bound on the table gradient (rows x dim) for either path; zero on
    rows no token uses.  x_rows: the gathered rows of every token (binary64)."""
    dim = x_rows.shape[1]
    k = depth(dim)
    tol = np.zeros((rows, dim))
    if idx.size == 0:
        return tol
    urows, first, counts, S, A = row_sums(idx, dy)
    xu = x_rows[first]
    _, _, r, xh = E.layer_norm_rows(xu, gamma, beta, eps)
    r = r[:, None]
    mabs_x = np.abs(xu).mean(axis=1, keepdims=True)
    c = counts[:, None].astype(np.float64)
    if grouped:
        dx = r * (S * gamma - (S * gamma).mean(axis=1, keepdims=True)
                  - xh * (S * gamma * xh).mean(axis=1, keepdims=True))
        t = map_tol(S, gamma, xh, r, mabs_x, k)
        if not exact_sums:
            d = sum_depth(counts)[:, None].astype(np.float64)
            t = t + 2 * map_abs(d * U * A, gamma, xh, r)
        t = t + 2 * U * (abs(base) + np.abs(dx))
    else:
        # every token's map bound and |dx| summed per row
        _, _, rt, xht = E.layer_norm_rows(x_rows, gamma, beta, eps)
        rt = rt[:, None]
        mx = np.abs(x_rows).mean(axis=1, keepdims=True)
        dyt = np.asarray(dy, np.float64)
        per_tok = map_tol(dyt, gamma, xht, rt, mx, k)
        gt = dyt * gamma
        dxt = rt * (gt - gt.mean(axis=1, keepdims=True)
                    - xht * (gt * xht).mean(axis=1, keepdims=True))
        order = np.argsort(idx, kind="stable")
        _, starts = np.unique(idx[order], return_index=True)
        summed = np.add.reduceat(per_tok[order], starts, axis=0)
        absdx = np.add.reduceat(np.abs(dxt[order]), starts, axis=0)
        t = summed + 2 * U * c * (abs(base) + absdx)
    tol[urows] = t
    return tol


def backward_ref_and_tol(x_rows, idx, rows, gamma, beta, dy, eps, base=0.0, grouped=None,
                         exact_sums=False):
    """Oracle gradients and per-element bounds for dweight (accumulated onto a table
    holding ``base``), dgamma and dbeta.  ``grouped`` defaults to the path the width
    takes; ``exact_sums`` declares upstream values whose binary32 token sums are exact."""
    dim = x_rows.shape[1]
    k = depth(dim)
    if grouped is None:
        grouped = grouped_path(dim)
    _, mean, rstd, xh = E.layer_norm_rows(x_rows, gamma, beta, eps)
    table = np.zeros((rows, dim))
    table[idx] = x_rows
    dw, dg, db = E.stable_embedding_backward(table, idx, gamma, beta, dy, eps)
    dw_tol = dweight_tol(x_rows, idx, rows, gamma, beta, dy, eps, base, grouped, exact_sums)
    n = idx.size
    r = rstd[:, None]
    mabs_x = np.abs(x_rows).mean(axis=1, keepdims=True)
    dxh_tol = (k / 2 + 8) * U * np.abs(xh) + (k + 1) * U * mabs_x * r
    dg_tol = 2 * ((np.abs(dy) * (dxh_tol + U * np.abs(xh))).sum(axis=0)
                  + (n + 8) * U * np.abs(dy * xh).sum(axis=0))
    db_tol = 2 * (n + 8) * U * np.abs(dy).sum(axis=0)
    return dw, dg, db, dw_tol, dg_tol, db_tol


def assert_within(got, want, tol, what):
    err = np.abs(got - want)
    bad = np.nonzero(~(err <= tol))
    assert bad[0].size == 0, (f"{what}: {bad[0].size} elements beyond the bound, worst ratio "
                              f"{np.max(err / np.maximum(tol, 1e-300)):.3g}")


def dyadic_upstream(rng, ntok, dim, max_k=64):
    """Upstream rows k * 2^-8 with integer |k| <= max_k (exact in bf16): for up to
    2^24 / max_k tokens on one row every binary32 partial sum is an exact multiple of
    2^-8 below 2^16, so the summation order cannot change a table row's sum."""
    return rng.integers(-max_k, max_k + 1, (ntok, dim)).astype(np.float64) * 2.0 ** -8
