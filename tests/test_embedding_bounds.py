"""CPU pins of the Stable Embedding table-gradient bound (tests/embedding_bounds.py).

The GPU tests accept a table-gradient row when it lies within this bound of the
oracle's.  These tests show the bound can fail where the grouped backward could go
wrong: on heavy rows (517 tokens, and 6,000, about as many as the most frequent id of
the 65,536-token Zipf batch) a row missing one token's gradient, or holding one twice,
or left at zero, lies outside it.  They also show it is not too tight: binary32
emulations of the kernels' arithmetic on either path (chunk-wise token sums, then one
LayerNorm backward; or one backward per token scattered in any order) stay inside it.
"""

import os
import re

import numpy as np
import pytest

import embedding_bounds as B
from oracle import embedding as E
from oracle import f32_to_bf16_rne

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
F = np.float32


def test_chunk_size_matches_the_kernels():
    src = open(os.path.join(ROOT, "block_wise_bit_adam8bit_amd", "csrc",
                            "stable_embedding.hip")).read()
    m = re.search(r"constexpr int kSegChunk = (\d+);", src)
    assert m and int(m.group(1)) == B.CHUNK


def test_sum_depth():
    assert list(B.sum_depth([0, 1, 2, 32, 33], chunk=None)) == [0, 0, 1, 31, 32]
    # a run inside one chunk is a plain sequential sum
    assert list(B.sum_depth([1, 5, 32])) == [0, 4, 31]
    # longer runs: a partial of at most 31 roundings, then one per further chunk
    assert int(B.sum_depth(33)) == 32 and int(B.sum_depth(6000)) == 31 + 188
    assert np.all(B.sum_depth(np.arange(1, 70000)) <= np.arange(0, 69999))


def _case(c, dim, seed, dyadic=False):
    """A 5-row table; row 1 is used by c tokens, rows 0, 2, 3 by a few, row 4 by none;
    tokens in random order.  Upstream rows bf16 N(0, 1), or on the dyadic grid."""
    rng = np.random.default_rng(seed)
    rows = 5
    w = rng.uniform(-0.05, 0.05, (rows, dim)).astype(F)
    w[0] += 3.0
    gamma = rng.normal(1.0, 0.25, dim).astype(F).astype(np.float64)
    beta = rng.normal(0.0, 0.1, dim).astype(F).astype(np.float64)
    idx = rng.permutation(np.concatenate([np.full(c, 1), [0, 0, 2, 3, 3, 3]])).astype(np.int64)
    if dyadic:
        dy = B.dyadic_upstream(rng, idx.size, dim)
    else:
        dy = (f32_to_bf16_rne(rng.normal(0, 1, (idx.size, dim)).astype(F))
              .astype(np.uint32) << np.uint32(16)).view(F).astype(np.float64)
    x = w.astype(np.float64)[idx]
    return w, idx, rows, gamma, beta, dy, x


def _one_token_dx(w, idx, gamma, beta, dy, t, eps=1e-5):
    return E.stable_embedding_backward(w.astype(np.float64), idx[t:t + 1], gamma, beta,
                                       dy[t:t + 1], eps)[0][idx[t]]


@pytest.mark.parametrize("c,dyadic,min_frac", [(517, False, 0.9), (6000, False, 0.45),
                                               (6000, True, 0.95)])
def test_bound_rejects_a_lost_or_repeated_token(c, dyadic, min_frac):
    w, idx, rows, gamma, beta, dy, x = _case(c, 4096, seed=c + dyadic)
    rdw, _, _, tdw, _, _ = B.backward_ref_and_tol(x, idx, rows, gamma, beta, dy, 1e-5,
                                                  exact_sums=dyadic)
    t = int(np.nonzero(idx == 1)[0][c // 2])
    one = _one_token_dx(w, idx, gamma, beta, dy, t)
    for wrong, what in ((rdw[1] - one, "one token lost"), (rdw[1] + one, "one token twice")):
        frac = np.mean(np.abs(wrong - rdw[1]) > tdw[1])
        assert frac > min_frac, f"{what}: only {frac:.3f} of the row's elements fail the bound"
    # a row left at zero fails everywhere the true gradient is not tiny
    assert np.mean(np.abs(rdw[1]) > tdw[1]) > 0.99
    # the lightly used rows too
    for r in (0, 2, 3):
        tr = int(np.nonzero(idx == r)[0][0])
        one = _one_token_dx(w, idx, gamma, beta, dy, tr)
        assert np.mean(np.abs(one) > tdw[r]) > 0.99
    assert not tdw[4].any()


def _rowsum(v):
    """binary32 row sum as the kernels take it: per lane (element i*64 + l on lane l)
    one after another, then halving across the 64 lanes."""
    n = -(-v.size // 64) * 64
    lanes = np.zeros(n, F)
    lanes[: v.size] = v
    s = np.zeros(64, F)
    for row in lanes.reshape(-1, 64):
        s = (s + row).astype(F)
    while s.size > 1:
        s = (s[: s.size // 2] + s[s.size // 2:]).astype(F)
    return s[0]


def _emulate_grouped(w, idx, gamma, beta, dy, eps, base, chunk, rng):
    """binary32 emulation of the grouped path: tokens sorted by row (a random offset of
    the first run into its chunk), each row's upstream rows summed one after another
    within chunks of `chunk` sorted tokens, the chunk partials in chunk order, then one
    LayerNorm backward with row sums per lane (64 lanes) and then across lanes."""
    rows, dim = w.shape
    out = np.full((rows, dim), F(base), F)
    order = np.argsort(idx, kind="stable")
    pos0 = int(rng.integers(0, chunk))           # sorted position of the first token
    g32 = gamma.astype(F)
    p = pos0
    for r in np.unique(idx):
        toks = order[idx[order] == r]
        parts, cur = [], F(0) * np.zeros(dim, F)
        for j, t in enumerate(toks):
            cur = (cur + dy[t].astype(F)).astype(F)
            if (p + j + 1) % chunk == 0 or j == toks.size - 1:
                parts.append(cur)
                cur = np.zeros(dim, F)
        acc = parts[0]
        for q in parts[1:]:
            acc = (acc + q).astype(F)
        p += toks.size
        x = w[r].astype(np.float64)
        mu = F(x.mean())
        rs = F(1.0 / np.sqrt(((x - x.mean()) ** 2).mean() + eps))
        x32 = w[r].astype(F)
        xh = ((x32 - mu) * rs).astype(F)
        gg = (acc * g32).astype(F)
        m1 = F(_rowsum(gg) / F(dim))
        m2 = F(_rowsum((gg * xh).astype(F)) / F(dim))
        d = (rs * (((acc * g32).astype(F) - m1).astype(F) - (xh * m2).astype(F))).astype(F)
        out[r] = (out[r] + d).astype(F)
    return out


@pytest.mark.parametrize("c,dyadic", [(517, False), (6000, False), (6000, True)])
def test_binary32_emulation_of_the_grouped_path_is_inside(c, dyadic):
    rng = np.random.default_rng(7)
    w, idx, rows, gamma, beta, dy, x = _case(c, 4096, seed=100 + c + dyadic, dyadic=dyadic)
    rdw, _, _, tdw, _, _ = B.backward_ref_and_tol(x, idx, rows, gamma, beta, dy, 1e-5,
                                                  base=0.5, exact_sums=dyadic)
    got = _emulate_grouped(w, idx, gamma, beta, dy, 1e-5, 0.5, B.CHUNK, rng)
    ratio = np.abs(got.astype(np.float64) - 0.5 - rdw) / np.maximum(tdw, 1e-300)
    used = np.unique(idx)
    assert ratio[used].max() < 0.5, ratio[used].max()


def test_binary32_emulation_of_the_element_path_is_inside():
    """Widths off the vector path: one backward per token in binary32, scattered onto
    the table in a random order."""
    rng = np.random.default_rng(8)
    dim = 1001
    w, idx, rows, gamma, beta, dy, x = _case(300, dim, seed=9)
    rdw, _, _, tdw, _, _ = B.backward_ref_and_tol(x, idx, rows, gamma, beta, dy, 1e-5,
                                                  base=0.5, grouped=False)
    out = np.full((rows, dim), F(0.5), F)
    g32 = gamma.astype(F)
    for t in rng.permutation(idx.size):
        xr = w[idx[t]].astype(np.float64)
        mu = F(xr.mean())
        rs = F(1.0 / np.sqrt(((xr - xr.mean()) ** 2).mean() + 1e-5))
        xh = ((w[idx[t]] - mu) * rs).astype(F)
        gg = (dy[t].astype(F) * g32).astype(F)
        m1 = F(_rowsum(gg) / F(dim))
        m2 = F(_rowsum((gg * xh).astype(F)) / F(dim))
        d = (rs * ((gg - m1).astype(F) - (xh * m2).astype(F))).astype(F)
        out[idx[t]] = (out[idx[t]] + d).astype(F)
    ratio = np.abs(out.astype(np.float64) - 0.5 - rdw) / np.maximum(tdw, 1e-300)
    assert ratio[np.unique(idx)].max() < 0.5
