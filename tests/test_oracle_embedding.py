"""Pins for the Stable Embedding oracle (CPU only).

The summary page (§2 "Stable Embedding Layer") fixes Xavier-uniform initialisation
and a layer normalisation after the lookup; the YaLM training page fixes a
LayerNorm right after the embedding, computed in fp32.  Checks: the generator's
published known-answer values, torch.nn.init's Xavier rule, the uniform law's
moments, torch's layer_norm and autograd in binary64, LayerNorm invariants, and
central finite differences of the forward for the backward.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import embedding as E

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")


def test_philox_known_answers():
    for vec in json.load(open(GOLDEN))["vectors"]:
        ctr = np.array([int(w, 16) for w in vec["ctr"]], np.uint32)
        key = np.array([int(w, 16) for w in vec["key"]], np.uint32)
        want = np.array([int(w, 16) for w in vec["out"]], np.uint32)
        assert np.array_equal(E.philox4x32_10(ctr, key), want)
        # batched evaluation gives the same words
        got = E.philox4x32_10(np.stack([ctr, ctr]), np.stack([key, key]))
        assert np.array_equal(got[1], want)


def test_uniform01_grid_and_range():
    w = np.array([0, 0xFF, 0x100, 0x80000000, 0xFFFFFFFF], np.uint32)
    u = E.uniform01(w)
    assert u.dtype == np.float32
    assert list(u) == [0.0, 0.0, 2.0 ** -24, 0.5, 1.0 - 2.0 ** -24]


@pytest.mark.parametrize("rows,dim", [(32000, 4096), (50257, 2048), (7, 5), (1, 1)])
def test_xavier_bound_matches_torch_rule(rows, dim):
    """torch.nn.init.xavier_uniform_ draws from U(-b, b) with b = gain * sqrt(6 /
    (fan_in + fan_out)) and its own fan convention for a 2-D [rows, dim] tensor."""
    fan_in, fan_out = torch.nn.init._calculate_fan_in_and_fan_out(torch.empty(rows, dim))
    b = torch.nn.init.calculate_gain("linear") * np.sqrt(6.0 / (fan_in + fan_out))
    assert E.xavier_bound(rows, dim) == np.float32(b)


def test_xavier_table_moments_and_layout():
    rows, dim, seed = 1000, 777, 1234
    w = E.xavier_uniform(rows, dim, seed)
    a = E.xavier_bound(rows, dim)
    assert w.shape == (rows, dim) and w.dtype == np.float32
    assert np.all(np.abs(w) <= a)
    n = w.size
    # U(-a, a): mean 0, variance a^2 / 3 (6 standard errors)
    assert abs(w.mean()) < 6 * a / np.sqrt(3 * n)
    var = (w.astype(np.float64) ** 2).mean()
    assert abs(var - a * a / 3) < 6 * a * a * np.sqrt(4 / 45 / n)
    # element e is word e % 4 of counter block e // 4
    e = 4 * 12345 + 2
    words = E.philox4x32_10(np.array([12345, 0, 0, 0], np.uint32), np.array([seed, 0], np.uint32))
    u = E.uniform01(words[2])
    assert w.reshape(-1)[e] == np.float32(a * ((np.float32(2) * u) - np.float32(1)))
    # another seed gives another table; the same seed the same one
    assert not np.array_equal(w, E.xavier_uniform(rows, dim, seed + 1))
    assert np.array_equal(w, E.xavier_uniform(rows, dim, seed))


def _case(rng, rows=50, dim=96, ntok=40):
    w = rng.uniform(-0.1, 0.1, (rows, dim))
    idx = rng.integers(0, rows, ntok)
    idx[:6] = idx[0]                           # repeated rows
    gamma = rng.normal(1.0, 0.3, dim)
    beta = rng.normal(0.0, 0.2, dim)
    return w, idx, gamma, beta


def test_forward_matches_torch_layer_norm():
    rng = np.random.default_rng(0)
    w, idx, gamma, beta = _case(rng)
    y, mean, rstd = E.stable_embedding_forward(w, idx, gamma, beta, 1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(w[idx]), (w.shape[1],),
                                         torch.from_numpy(gamma), torch.from_numpy(beta), 1e-5)
    assert np.allclose(y, ref.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(mean, w[idx].mean(axis=1), rtol=0, atol=1e-15)


def test_forward_invariants():
    rng = np.random.default_rng(1)
    w, idx, _, _ = _case(rng)
    ones, zeros = np.ones(w.shape[1]), np.zeros(w.shape[1])
    y, _, _ = E.stable_embedding_forward(w, idx, ones, zeros, 0.0)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((y ** 2).mean(axis=1), 1, atol=1e-12)
    # shifting a row by a constant or scaling it (eps = 0) changes nothing
    y2, _, _ = E.stable_embedding_forward(3.0 * w + 7.0, idx, ones, zeros, 0.0)
    assert np.allclose(y, y2, atol=1e-9)
    # gamma and beta act per column
    g = rng.normal(size=w.shape[1])
    b = rng.normal(size=w.shape[1])
    y3, _, _ = E.stable_embedding_forward(w, idx, g, b, 0.0)
    assert np.allclose(y3, y * g + b, atol=1e-12)
    with pytest.raises(IndexError):
        E.stable_embedding_forward(w, np.array([w.shape[0]]), ones, zeros)


def test_backward_central_differences():
    """Every gradient entry of a tiny case against (f(x + h) - f(x - h)) / 2h."""
    rng = np.random.default_rng(2)
    w, idx, gamma, beta = _case(rng, rows=6, dim=5, ntok=8)
    idx[:3] = 2
    eps = 1e-5
    dy = rng.normal(size=(idx.size, w.shape[1]))

    def loss(w_, g_, b_):
        y, _, _ = E.stable_embedding_forward(w_, idx, g_, b_, eps)
        return float((y * dy).sum())

    dw, dg, db = E.stable_embedding_backward(w, idx, gamma, beta, dy, eps)
    h = 1e-6
    for arr, grad in ((w, dw), (gamma, dg), (beta, db)):
        num = np.zeros_like(arr)
        for k in np.ndindex(arr.shape):
            old = arr[k]
            arr[k] = old + h
            fp = loss(w, gamma, beta)
            arr[k] = old - h
            fm = loss(w, gamma, beta)
            arr[k] = old
            num[k] = (fp - fm) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-7)
    # rows no token uses get no gradient
    unused = np.setdiff1d(np.arange(w.shape[0]), idx)
    assert not dw[unused].any()


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(3)
    w, idx, gamma, beta = _case(rng, rows=300, dim=256, ntok=500)
    dy = rng.normal(size=(idx.size, w.shape[1]))
    tw = torch.from_numpy(w).requires_grad_()
    tg = torch.from_numpy(gamma).requires_grad_()
    tb = torch.from_numpy(beta).requires_grad_()
    y = torch.nn.functional.layer_norm(torch.nn.functional.embedding(torch.from_numpy(idx), tw),
                                       (w.shape[1],), tg, tb, 1e-5)
    y.backward(torch.from_numpy(dy))
    dw, dg, db = E.stable_embedding_backward(w, idx, gamma, beta, dy, 1e-5)
    assert np.allclose(dw, tw.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dg, tg.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(db, tb.grad.numpy(), rtol=1e-10, atol=1e-12)
