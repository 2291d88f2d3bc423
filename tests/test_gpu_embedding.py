"""GPU parity of the Stable Embedding kernels against the oracle.

Initialisation is compared bit for bit.  The forward and backward passes compute in
binary32 and are compared with the binary64 oracle within bounds derived from their
arithmetic (tests/embedding_bounds.py, whose CPU tests show the table-gradient bound
rejects a row that lost or repeated one token even at 6,000 tokens per row).
dgamma and dbeta are bounded for any summation order by (N + 8) u times the sum of
magnitudes.
"""

import numpy as np
import pytest
import torch

import workloads
from embedding_bounds import (U, assert_within, backward_ref_and_tol, depth, dyadic_upstream,
                              forward_tol)
from oracle import embedding as E
from oracle import f32_to_bf16_rne

pytestmark = pytest.mark.gpu
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_wise_bit_adam8bit_amd as q
    torch.cuda.set_device(0)
    return q


def to_dev(a, dt):
    """float array (already representable in dt) -> device tensor of dt."""
    if dt == "bf16":
        return torch.from_numpy(f32_to_bf16_rne(np.asarray(a, np.float32)).view(np.int16)) \
            .cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


# ------------------------------------------------------------------ initialisation


@pytest.mark.parametrize("rows,dim", [(1000, 96), (7, 5), (3, 1), (1, 4099)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_xavier_init_bit_exact(q, rows, dim, dt):
    say(f"xavier {rows}x{dim} {dt}")
    for seed in (0, 123456789012345):
        w = torch.empty(rows, dim, dtype=DT[dt], device="cuda")
        q.qopt_embedding_xavier_init(w, seed)
        want = E.xavier_uniform(rows, dim, seed)
        if dt == "bf16":
            got = w.view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(got, f32_to_bf16_rne(want))
        else:
            assert np.array_equal(w.cpu().numpy().view(np.uint32), want.view(np.uint32))


# ------------------------------------------------------------------ forward / backward


SHAPES = [(500, 4096), (300, 2048), (200, 1000), (100, 768), (64, 96), (50, 4), (30, 5),
          (40, 4100), (20, 6001)]


def _inputs(rows, dim, ntok, seed):
    rng = np.random.default_rng(seed)
    w = rng.uniform(-0.05, 0.05, (rows, dim)).astype(np.float32)
    w[0] += 3.0                                   # one row with a large offset
    idx = rng.integers(0, rows, ntok).astype(np.int64)
    idx[: min(8, ntok)] = idx[0]                  # a repeated row
    gamma = rng.normal(1.0, 0.25, dim).astype(np.float32)
    beta = rng.normal(0.0, 0.1, dim).astype(np.float32)
    dy = rng.normal(0.0, 1.0, (ntok, dim)).astype(np.float32)
    return w, idx, gamma, beta, dy


@pytest.mark.parametrize("rows,dim", SHAPES)
@pytest.mark.parametrize("wdt,odt", [("f32", "f32"), ("f32", "bf16"), ("bf16", "bf16"),
                                     ("bf16", "f32")])
def test_forward_and_backward(q, rows, dim, wdt, odt):
    ntok = 300
    say(f"stable embedding {rows}x{dim} tokens {ntok} {wdt}->{odt}")
    w, idx, gamma, beta, dy = _inputs(rows, dim, ntok, seed=rows * 7 + dim)
    if wdt == "bf16":
        w = (f32_to_bf16_rne(w).astype(np.uint32) << np.uint32(16)).view(np.float32)
    if odt == "bf16":
        dy = (f32_to_bf16_rne(dy).astype(np.uint32) << np.uint32(16)).view(np.float32)
    eps = 1e-5
    tw, tidx = to_dev(w, wdt), torch.from_numpy(idx).cuda()
    tg, tb = to_dev(gamma, "f32"), to_dev(beta, "f32")
    out, mean, rstd = q.qopt_stable_embedding_forward(tw, tidx, tg, tb, eps, DT[odt])
    x = w.astype(np.float64)[idx]
    y, mref, rref, tol = forward_tol(x, gamma.astype(np.float64), beta.astype(np.float64), eps, odt)
    torch.cuda.synchronize()
    assert out.shape == (ntok, dim) and out.dtype == DT[odt]
    assert_within(host(out), y, tol, "forward output")
    k = depth(dim)
    assert_within(host(mean), mref, 2 * (k + 1) * U * np.abs(x).mean(axis=1) + 1e-30, "mean")
    assert_within(host(rstd), rref, 2 * (k / 2 + 7) * U * rref, "rstd")

    tdy = to_dev(dy, odt)
    dw0 = torch.full((rows, dim), 0.5, dtype=torch.float32, device="cuda")
    dw, dg, db = q.qopt_stable_embedding_backward(tw, tidx, tg, mean, rstd, tdy, dweight=dw0)
    rdw, rdg, rdb, tdw, tdg, tdb = backward_ref_and_tol(x, idx, rows, gamma.astype(np.float64),
                                                        beta.astype(np.float64),
                                                        dy.astype(np.float64), eps, base=0.5)
    torch.cuda.synchronize()
    assert dw.data_ptr() == dw0.data_ptr()
    assert_within(host(dw) - 0.5, rdw, tdw, "dweight (accumulated onto 0.5)")
    assert_within(host(dg), rdg, tdg, "dgamma")
    assert_within(host(db), rdb, tdb, "dbeta")
    # gamma and beta gradients are summed in a fixed order: a second run is identical;
    # so is the table gradient on the grouped (vector) path
    dw_a, dg2, db2 = q.qopt_stable_embedding_backward(tw, tidx, tg, mean, rstd, tdy)
    dw_b, _, _ = q.qopt_stable_embedding_backward(tw, tidx, tg, mean, rstd, tdy)
    assert torch.equal(dg, dg2) and torch.equal(db, db2)
    if dim % 4 == 0 and dim <= 4096:
        assert torch.equal(dw_a, dw_b)


RUN_LAYOUTS = [
    [1, 31, 32, 33, 63, 64, 65, 96, 200, 1, 2, 31],   # runs ending on and beside 32-token marks
    [517],                                              # one row takes every token
    [300, 217],                                         # two long runs, the last ending at the end
    [1] * 40 + [140] + [1] * 30,                        # a long run among single tokens
]


@pytest.mark.parametrize("dim", [256, 4096])
@pytest.mark.parametrize("lengths", RUN_LAYOUTS + [[3, 6000, 5, 2000, 1]])
@pytest.mark.parametrize("upstream", ["normal", "dyadic"])
def test_run_layouts_across_chunks(q, dim, lengths, upstream):
    """Sorted runs of chosen lengths, so that runs start and end on, just before and just
    after chunk boundaries of any power-of-two chunk size up to 64, span many chunks,
    or cover the whole batch: every table-gradient row, dgamma and dbeta against the
    oracle.  Upstream rows are bf16 N(0, 1), or dyadic values whose binary32 token sums
    are exact in any order, so that only the count-independent bound of one LayerNorm
    backward per row remains (a run missing one of 6,000 tokens then fails in nearly
    every element)."""
    ntok = sum(lengths)
    say(f"run layouts dim {dim} {upstream} lengths {lengths[:6]}... ({len(lengths)} runs, "
        f"{ntok} tokens)")
    rows = len(lengths) + 3
    rng = np.random.default_rng(dim + ntok)
    w = rng.uniform(-0.05, 0.05, (rows, dim)).astype(np.float32)
    gamma = rng.normal(1.0, 0.25, dim).astype(np.float32)
    beta = rng.normal(0.0, 0.1, dim).astype(np.float32)
    # run r (in sorted order) is row r + 1; tokens in random order
    idx = rng.permutation(np.repeat(np.arange(1, len(lengths) + 1), lengths)).astype(np.int64)
    if upstream == "dyadic":
        dy = dyadic_upstream(rng, ntok, dim).astype(np.float32)
    else:
        dy = (f32_to_bf16_rne(rng.normal(0.0, 1.0, (ntok, dim)).astype(np.float32))
              .astype(np.uint32) << np.uint32(16)).view(np.float32)
    tw, tidx = to_dev(w, "f32"), torch.from_numpy(idx).cuda()
    tg, tb = to_dev(gamma, "f32"), to_dev(beta, "f32")
    out, mean, rstd = q.qopt_stable_embedding_forward(tw, tidx, tg, tb, 1e-5, torch.bfloat16)
    dw, dg, db = q.qopt_stable_embedding_backward(tw, tidx, tg, mean, rstd, to_dev(dy, "bf16"))
    x = w.astype(np.float64)[idx]
    rdw, rdg, rdb, tdw, tdg, tdb = backward_ref_and_tol(x, idx, rows, gamma.astype(np.float64),
                                                        beta.astype(np.float64),
                                                        dy.astype(np.float64), 1e-5,
                                                        exact_sums=upstream == "dyadic")
    torch.cuda.synchronize()
    assert_within(host(dw), rdw, tdw, "dweight")
    assert not host(dw)[0].any() and not host(dw)[-2:].any()   # rows no token uses
    assert_within(host(dg), rdg, tdg, "dgamma")
    assert_within(host(db), rdb, tdb, "dbeta")


def test_misaligned_views_take_the_element_path(q):
    rows, dim, ntok = 64, 256, 100
    w, idx, gamma, beta, dy = _inputs(rows, dim, ntok, seed=9)
    buf = torch.zeros(rows * dim + 1, dtype=torch.float32, device="cuda")
    tw = buf[1:].view(rows, dim)
    tw.copy_(torch.from_numpy(w).cuda())
    out, mean, rstd = q.qopt_stable_embedding_forward(tw, torch.from_numpy(idx).cuda(),
                                                      to_dev(gamma, "f32"), to_dev(beta, "f32"))
    y, _, _, tol = forward_tol(w.astype(np.float64)[idx], gamma.astype(np.float64),
                               beta.astype(np.float64), 1e-5, "f32")
    torch.cuda.synchronize()
    assert_within(host(out), y, tol, "forward output (unaligned table)")


def test_runs_on_the_callers_stream(q):
    """Forward and backward go on the caller's current stream: on a side stream
    (default priority) queued behind long matrix products and the copies that fill
    their inputs, they must see those inputs and give the same bits as on the default
    stream (both passes are deterministic)."""
    rows, dim, ntok = 300, 2048, 1500
    w_h, idx_h, g_h, b_h = _inputs(rows, dim, ntok, 91)[:4]
    w, gamma, beta = to_dev(w_h, "f32"), to_dev(g_h, "f32"), to_dev(b_h, "f32")
    idx = torch.from_numpy(idx_h).cuda()
    dy_h = np.random.default_rng(92).normal(0.0, 1.0, (ntok, dim)).astype(np.float32)
    dy = to_dev(dy_h, "bf16")
    out0, mean0, rstd0 = q.qopt_stable_embedding_forward(w, idx, gamma, beta, out_dtype=torch.bfloat16)
    dw0, dg0, db0 = q.qopt_stable_embedding_backward(w, idx, gamma, mean0, rstd0, dy)
    torch.cuda.synchronize()
    idx_s, dy_s = torch.zeros_like(idx), torch.zeros_like(dy)
    side = torch.cuda.Stream()
    say(f"side stream embedding rows={rows} dim={dim} ntok={ntok}")
    with torch.cuda.stream(side):
        a = torch.full((4096, 4096), 1.0 / 4096, device="cuda")  # a @ a == a
        for _ in range(12):
            a = a @ a
        idx_s.copy_(idx)
        dy_s.copy_(dy)
        out1, mean1, rstd1 = q.qopt_stable_embedding_forward(w, idx_s, gamma, beta,
                                                             out_dtype=torch.bfloat16)
        dw1, dg1, db1 = q.qopt_stable_embedding_backward(w, idx_s, gamma, mean1, rstd1, dy_s)
    side.synchronize()
    for nm, x0, x1 in [("out", out0, out1), ("mean", mean0, mean1), ("rstd", rstd0, rstd1),
                       ("dweight", dw0, dw1), ("dgamma", dg0, dg1), ("dbeta", db0, db1)]:
        assert torch.equal(x0.view(torch.int16) if x0.dtype == torch.bfloat16 else x0.view(torch.int32),
                           x1.view(torch.int16) if x1.dtype == torch.bfloat16 else x1.view(torch.int32)), nm


def test_bad_indices_and_empty_batches(q):
    rows, dim = 16, 512
    w, _, gamma, beta, _ = _inputs(rows, dim, 4, seed=10)
    tw, tg, tb = to_dev(w, "f32"), to_dev(gamma, "f32"), to_dev(beta, "f32")
    idx = torch.tensor([3, -1, 16, 5, 1 << 40], dtype=torch.int64, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, mean, rstd = q.qopt_stable_embedding_forward(tw, idx, tg, tb, bad_count=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 3
    o = out.cpu().numpy()
    assert np.isnan(o[[1, 2, 4]]).all() and np.isfinite(o[[0, 3]]).all()
    dy = torch.ones(5, dim, device="cuda")
    dw, dg, db = q.qopt_stable_embedding_backward(tw, idx, tg, mean, rstd, dy)
    torch.cuda.synchronize()
    touched = np.nonzero(np.abs(dw.cpu().numpy()).sum(axis=1))[0]
    assert set(touched.tolist()) <= {3, 5}
    assert np.allclose(db.cpu().numpy(), 2.0)           # only the two valid tokens
    # no tokens: outputs empty, gamma / beta gradients zero, table gradient untouched
    e = torch.empty(0, dtype=torch.int64, device="cuda")
    out0, m0, r0 = q.qopt_stable_embedding_forward(tw, e, tg, tb)
    assert out0.shape == (0, dim)
    dw0 = torch.full((rows, dim), 2.0, device="cuda")
    _, dg0, db0 = q.qopt_stable_embedding_backward(tw, e, tg, m0, r0,
                                                   torch.empty(0, dim, device="cuda"), dweight=dw0)
    torch.cuda.synchronize()
    assert not dg0.any() and not db0.any() and bool((dw0 == 2.0).all())


def test_module_autograd_against_oracle(q):
    """StableEmbedding: Xavier-initialised table, LayerNorm output, gradients of all
    three parameters through torch autograd; out-of-range ids raise."""
    rows, dim, seed = 1000, 1024, 77
    m = q.StableEmbedding(rows, dim, seed=seed, out_dtype=torch.bfloat16)
    assert np.array_equal(m.weight.detach().cpu().numpy(), E.xavier_uniform(rows, dim, seed))
    ids = workloads.zipf_token_ids(4 * 128, rows, seed=3).reshape(4, 128)
    tids = torch.from_numpy(ids).cuda()
    with torch.no_grad():
        m.norm_weight.copy_(torch.linspace(0.5, 1.5, dim))
        m.norm_bias.copy_(torch.linspace(-0.1, 0.1, dim))
    y = m(tids)
    assert y.shape == (4, 128, dim) and y.dtype == torch.bfloat16
    dy = torch.randn(4, 128, dim, device="cuda", generator=torch.Generator("cuda").manual_seed(5))
    dy = dy.bfloat16()
    y.backward(dy)
    w = E.xavier_uniform(rows, dim, seed).astype(np.float64)
    gamma = np.linspace(0.5, 1.5, dim, dtype=np.float32).astype(np.float64)
    beta = np.linspace(-0.1, 0.1, dim, dtype=np.float32).astype(np.float64)
    idx = ids.reshape(-1)
    yref, _, _, tol = forward_tol(w[idx], gamma, beta, 1e-5, "bf16")
    assert_within(host(y).reshape(-1, dim), yref, tol, "module output")
    rdw, rdg, rdb, tdw, tdg, tdb = backward_ref_and_tol(w[idx], idx, rows, gamma, beta,
                                                        host(dy).reshape(-1, dim), 1e-5)
    assert_within(host(m.weight.grad), rdw, tdw, "weight grad")
    assert_within(host(m.norm_weight.grad), rdg, tdg, "gamma grad")
    assert_within(host(m.norm_bias.grad), rdb, tdb, "beta grad")
    with pytest.raises(IndexError):
        m(torch.tensor([rows], device="cuda"))


def test_full_size_sampled(q):
    """The Llama-7B embedding shape with 65,536 Zipf-distributed tokens, as the bench
    runs it: sampled tokens' outputs, the table-gradient rows of every id used by at
    least 500 tokens plus sampled ones against the oracle, and gamma / beta gradients
    over all tokens."""
    cfg = workloads.EMBED7B
    rows, dim, ntok = cfg["rows"], cfg["dim"], cfg["ntokens"]
    say(f"full size {rows}x{dim}, {ntok} tokens")
    seed = 41
    tw = torch.empty(rows, dim, device="cuda")
    q.qopt_embedding_xavier_init(tw, seed)
    ids = workloads.zipf_token_ids(ntok, rows, seed=7)
    tids = torch.from_numpy(ids).cuda()
    tg = torch.ones(dim, device="cuda")
    tb = torch.zeros(dim, device="cuda")
    out, mean, rstd = q.qopt_stable_embedding_forward(tw, tids, tg, tb, 1e-5, torch.bfloat16)
    g = torch.Generator("cuda").manual_seed(8)
    tdy = torch.randn(ntok, dim, device="cuda", generator=g).bfloat16()
    dw, dg, db = q.qopt_stable_embedding_backward(tw, tids, tg, mean, rstd, tdy)
    torch.cuda.synchronize()
    w = tw.cpu().numpy().astype(np.float64)
    assert np.array_equal(tw.cpu().numpy(), E.xavier_uniform(rows, dim, seed))
    gamma, beta = np.ones(dim), np.zeros(dim)
    rng = np.random.default_rng(9)
    toks = np.unique(np.concatenate([[0, ntok - 1], rng.choice(ntok, 512, replace=False)]))
    y, _, _, tol = forward_tol(w[ids[toks]], gamma, beta, 1e-5, "bf16")
    assert_within(host(out[torch.from_numpy(toks).cuda()]), y, tol, "sampled outputs")
    dy = host(tdy)
    # table-gradient rows: every row with at least 500 tokens (about a quarter of the
    # batch), a rare one and random ones
    uniq, counts = np.unique(ids, return_counts=True)
    heavy = uniq[counts >= 500]
    assert heavy.size >= 10 and counts.max() > 5000
    pick = np.unique(np.concatenate([heavy, [uniq[np.argmin(counts)]],
                                     rng.choice(uniq, 20, replace=False)]))
    sel = np.nonzero(np.isin(ids, pick))[0]
    rdw, _, _, tdw, _, _ = backward_ref_and_tol(w[ids[sel]], ids[sel], rows, gamma, beta,
                                                dy[sel], 1e-5)
    assert_within(host(dw[torch.from_numpy(pick).cuda()]), rdw[pick], tdw[pick],
                  "sampled table-gradient rows")
    # gamma and beta gradients over all tokens, in chunks
    x_all = None
    rdg = np.zeros(dim)
    rdb = np.zeros(dim)
    tdg = np.zeros(dim)
    k = depth(dim)
    for s in range(0, ntok, 8192):
        x_all = w[ids[s:s + 8192]]
        _, _, r, xh = E.layer_norm_rows(x_all, gamma, beta, 1e-5)
        d = dy[s:s + 8192]
        rdg += (d * xh).sum(axis=0)
        rdb += d.sum(axis=0)
        dxh = (k / 2 + 8) * U * np.abs(xh) + (k + 1) * U * np.abs(x_all).mean(axis=1,
                                                                         keepdims=True) * r[:, None]
        tdg += 2 * ((np.abs(d) * (dxh + U * np.abs(xh))).sum(axis=0)
                    + (ntok + 8) * U * np.abs(d * xh).sum(axis=0))
    assert_within(host(dg), rdg, tdg, "dgamma")
    assert_within(host(db), rdb, 2 * (ntok + 8) * U * np.abs(dy).sum(axis=0), "dbeta")
