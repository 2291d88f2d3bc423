"""GPU parity of the fused 8-bit Adam kernel against the oracle.

The codes and block maxima must be bit-exact; parameters must agree within
|delta| <= 1e-6 * max(|p_ref|, lr) (and, since both sides round the same binary32
operations in the same order, they are expected to be bit-exact too).  Small cases
compare every element; the full-size parameter sets compare sampled blocks, whose
trajectories the oracle can run on their own because blocks are independent.
"""

import copy
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import BLOCK

pytestmark = pytest.mark.gpu
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_wise_bit_adam8bit_amd as q
    torch.cuda.set_device(0)
    return q


# ----------------------------------------------------------------- helpers


def to_dev(a, dtype):
    """numpy fp32 or bf16 bit patterns (uint16) -> device tensor of ``dtype``."""
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16).copy()).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def to_host(t, dtype):
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()  # fp32 values or uint8 codes


def host_state(n):
    nb = -(-n // BLOCK)
    return [np.zeros(n, np.uint8), np.zeros(n, np.uint8), np.zeros(nb, np.float32),
            np.zeros(nb, np.float32)]


def dev_state(n):
    nb = -(-n // BLOCK)
    return [torch.zeros(n, dtype=torch.uint8, device="cuda"),
            torch.zeros(n, dtype=torch.uint8, device="cuda"),
            torch.zeros(nb, dtype=torch.float32, device="cuda"),
            torch.zeros(nb, dtype=torch.float32, device="cuda")]


def assert_params(p_got, p_ref, pdt, lr, what=""):
    if pdt == "bf16":
        assert np.array_equal(p_got, p_ref), f"bf16 params differ {what}"
        return
    g = p_got.astype(np.float64)
    r = p_ref.astype(np.float64)
    err = np.abs(g - r)
    tol = 1e-6 * np.maximum(np.abs(r), lr)
    assert np.all(err <= tol), f"params beyond tolerance {what}: max err {err.max()}"
    assert np.array_equal(p_got.view(np.uint32), p_ref.view(np.uint32)), \
        f"params not bit-exact {what}: {np.count_nonzero(p_got != p_ref)} differ"


def assert_state(got, ref, what=""):
    names = ["m_codes", "v_codes", "m_absmax", "v_absmax"]
    for nm, a, b in zip(names, got, ref):
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        bad = np.nonzero(a != b)[0]
        assert bad.size == 0, f"{nm} differs {what} at {bad[:5]} ({bad.size} total)"


def host_grads(n, gdt, rng, scale=1e-3):
    g = rng.normal(0, scale, n).astype(np.float32)
    g[rng.choice(n, size=max(1, n // 500), replace=False)] *= 100
    return oracle.f32_to_bf16_rne(g) if gdt == "bf16" else g


def host_params(n, pdt, rng):
    p = rng.normal(0, 0.02, n).astype(np.float32)
    return oracle.f32_to_bf16_rne(p) if pdt == "bf16" else p


def run_small(q, sizes, pdt, gdt, steps, seed, hp=HP, views=None, grads=None):
    """Full-element parity over a list of tensors for several steps."""
    rng = np.random.default_rng(seed)
    grads = grads or host_grads
    hp_p = [host_params(n, pdt, rng) for n in sizes]
    hs = [host_state(n) for n in sizes]
    if views is None:
        dp = [to_dev(p, pdt) for p in hp_p]
        ds = [dev_state(n) for n in sizes]
    else:
        dp, ds = views(hp_p)
    for step in range(1, steps + 1):
        hg = [grads(n, gdt, rng) for n in sizes]
        dg = [to_dev(g, gdt) for g in hg]
        q.qopt_adam8bit_step([(dp[i], dg[i], *ds[i]) for i in range(len(sizes))],
                             step=step, **hp)
        for i, n in enumerate(sizes):
            out = oracle.adam8bit_step(hp_p[i], hg[i], *hs[i], step=step, param_dtype=pdt,
                                       grad_dtype=gdt, **hp)
            hp_p[i], hs[i] = out[0], list(out[1:])
        torch.cuda.synchronize()
        for i, n in enumerate(sizes):
            what = f"(tensor {i}, n={n}, step {step}, {pdt}/{gdt})"
            assert_state([t.cpu().numpy() for t in ds[i]], hs[i], what)
            assert_params(to_host(dp[i], pdt), hp_p[i], pdt, hp["lr"], what)


# ------------------------------------------------------------- small cases


def test_flat1m_ten_steps(q):
    """One fp32 tensor of 1,048,576 params, fp32 grads with 0.1 % outliers x100,
    10 steps from zero state: every element compared after every step."""
    p0, grads = workloads.flat1m()
    n = p0.size
    say(f"flat1m n={n}")
    p = torch.from_numpy(p0.copy()).cuda()
    st = dev_state(n)
    ref = [p0.copy(), *host_state(n)]
    for step, g in enumerate(grads, start=1):
        q.qopt_adam8bit_step([(p, torch.from_numpy(g).cuda(), *st)], step=step, **HP)
        out = oracle.adam8bit_step(ref[0], g, *ref[1:], step=step, **HP)
        ref = list(out)
        torch.cuda.synchronize()
        assert_state([t.cpu().numpy() for t in st], ref[1:], f"step {step}")
        assert_params(p.cpu().numpy(), ref[0], "f32", HP["lr"], f"step {step}")


@pytest.mark.parametrize("pdt,gdt", [("f32", "f32"), ("f32", "bf16"), ("bf16", "f32"),
                                     ("bf16", "bf16")])
def test_dtypes_and_tails(q, pdt, gdt):
    sizes = [1, 7, 2047, 2048, 2049, 50257, 3 * 2048 + 5, 17 * 2048]
    say(f"tails {pdt}/{gdt}")
    run_small(q, sizes, pdt, gdt, steps=3, seed=sum(map(ord, pdt + gdt)))


def test_many_tensors_span_several_launches(q):
    rng = np.random.default_rng(3)
    sizes = [int(s) for s in rng.integers(1, 6000, 130)]
    say(f"{len(sizes)} tensors")
    run_small(q, sizes, "f32", "bf16", steps=2, seed=4)


def test_misaligned_views(q):
    """Params, grads and codes as views at odd element offsets of flat buffers."""
    sizes = [3 * 2048 + 11, 2048, 5000]

    def views(hp_p):
        tot = sum(sizes) + 16
        pbuf = torch.zeros(tot, dtype=torch.float32, device="cuda")
        cbuf = torch.zeros(2 * tot, dtype=torch.uint8, device="cuda")
        dp, ds, off, coff = [], [], 1, 3
        for p, n in zip(hp_p, sizes):
            v = pbuf[off:off + n]
            v.copy_(torch.from_numpy(p).cuda())
            dp.append(v)
            nb = -(-n // BLOCK)
            ds.append([cbuf[coff:coff + n], cbuf[coff + tot:coff + tot + n],
                       torch.zeros(nb, dtype=torch.float32, device="cuda"),
                       torch.zeros(nb, dtype=torch.float32, device="cuda")])
            off += n + 1
            coff += n + 1
        return dp, ds

    say("misaligned views")
    run_small(q, sizes, "f32", "f32", steps=3, seed=5, views=views)


@pytest.mark.parametrize("pdt,gdt", [("f32", "bf16"), ("bf16", "bf16")])
def test_misaligned_pieces_inside_runs(q, pdt, gdt):
    """One launch of more blocks than the grid's waves take in whole runs, in which
    tensors that must take the element-wise path (parameters at odd element offsets)
    sit between aligned ones, so that runs of consecutive blocks pass from vector
    blocks to element-wise ones and back, and the next block a wave loads ahead is
    sometimes not a vector block."""
    sizes = [5 * 2048 + 11, 4000 * 2048, 2049, 4200 * 2048, 7]
    odd = {0, 2, 4}
    elt = torch.float32 if pdt == "f32" else torch.bfloat16

    def views(hp_p):
        tot = sum(sizes) + 2048 * len(sizes)
        pbuf = torch.zeros(tot, dtype=elt, device="cuda")
        dp, ds, off = [], [], 0
        for i, (p, n) in enumerate(zip(hp_p, sizes)):
            start = off + (1 if i in odd else 0)
            v = pbuf[start:start + n]
            v.copy_(to_dev(p, pdt))
            dp.append(v)
            ds.append(dev_state(n))
            off += -(-(n + 1) // 2048) * 2048
        return dp, ds

    say(f"misaligned pieces inside runs {pdt}/{gdt}")
    run_small(q, sizes, pdt, gdt, steps=2, seed=29, views=views)


@pytest.mark.parametrize("pdt,gdt", [("f32", "bf16"), ("bf16", "bf16")])
def test_rank_shares_step_independently(q, pdt, gdt):
    """Three ranks' shares (contiguous ranges of whole blocks of the flattened tensors,
    each stepped by its own call on views of the full tensors and block maxima) give
    the oracle's whole-tensor step, element for element."""
    sizes = [5 * 2048 + 5, 2048, 5000, 9 * 2048, 1, 2049, 4 * 2048 + 100]
    world = 3
    rng = np.random.default_rng(21)
    hp_p = [host_params(n, pdt, rng) for n in sizes]
    hs = [host_state(n) for n in sizes]
    dp = [to_dev(p, pdt) for p in hp_p]
    ds = [dev_state(n) for n in sizes]
    shares = [workloads.shard_pieces(sizes, world, r) for r in range(world)]
    # tensors 2 and 3 are split between ranks, one piece being tensor 2's ragged tail
    assert (2, 4096, 904) in shares[1] and sum(len(s) for s in shares) == len(sizes) + 2
    for step in range(1, 4):
        hg = [host_grads(n, gdt, rng) for n in sizes]
        dg = [to_dev(g, gdt) for g in hg]
        for r, pieces in enumerate(shares):
            items = []
            for i, e0, c in pieces:
                b0, nb = e0 // BLOCK, -(-c // BLOCK)
                items.append((dp[i][e0:e0 + c], dg[i][e0:e0 + c], ds[i][0][e0:e0 + c],
                              ds[i][1][e0:e0 + c], ds[i][2][b0:b0 + nb], ds[i][3][b0:b0 + nb]))
            q.qopt_adam8bit_step(items, step=step, **HP)
        for i in range(len(sizes)):
            out = oracle.adam8bit_step(hp_p[i], hg[i], *hs[i], step=step, param_dtype=pdt,
                                       grad_dtype=gdt, **HP)
            hp_p[i], hs[i] = out[0], list(out[1:])
        torch.cuda.synchronize()
        for i, n in enumerate(sizes):
            what = f"(tensor {i}, n={n}, step {step}, {world} shares, {pdt}/{gdt})"
            assert_state([t.cpu().numpy() for t in ds[i]], hs[i], what)
            assert_params(to_host(dp[i], pdt), hp_p[i], pdt, HP["lr"], what)


def _grads_max_at_position(n, gdt, rng):
    """Block b's largest gradient sits at element b % 2048 of the block (signs
    alternating), so over 2048 blocks the largest m and v of a block are held once
    by every lane in every slice."""
    nb = n // BLOCK
    g = rng.normal(0, 1e-4, n).astype(np.float32)
    b = np.arange(nb)
    g[b * BLOCK + b % BLOCK] = np.where(b % 2 == 0, 0.1, -0.1).astype(np.float32)
    return oracle.f32_to_bf16_rne(g) if gdt == "bf16" else g


@pytest.mark.parametrize("pdt,gdt", [("f32", "bf16"), ("bf16", "bf16")])
def test_block_max_at_every_position(q, pdt, gdt):
    """The block maxima of m and v (a reduction across the wave) are exact wherever
    in the block the maximum lies; fp32 and bf16 parameters keep v in different
    places (registers, LDS) until the maximum is known."""
    say(f"block max at every position {pdt}/{gdt}")
    run_small(q, [BLOCK * BLOCK], pdt, gdt, steps=2, seed=7, grads=_grads_max_at_position)


@pytest.mark.parametrize("hp", [dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8),
                                dict(lr=5e-2, beta1=0.5, beta2=0.75, eps=1e-6),
                                dict(lr=1e-4, beta1=0.95, beta2=0.9999, eps=0.0)])
def test_other_hyperparameters(q, hp):
    say(f"hyper-parameters {hp}")
    run_small(q, [2048 * 3 + 100], "f32", "f32", steps=4, seed=6, hp=hp)


@pytest.mark.parametrize("pdt,gdt", [("f32", "f32"), ("bf16", "bf16")])
def test_tiny_second_moments(q, pdt, gdt):
    """Gradients from 1e-30 to 1e-3 within and across blocks: second moments in
    (0, 2^-96), subnormal ones, exact zeros and ordinary ones, so both square-root
    branches of the kernel run, in the same wave and in separate waves."""
    def grads(n, gdt_, rng):
        mag = 10.0 ** rng.uniform(-30, -3, n)
        g = (rng.choice([-1.0, 1.0], n) * mag).astype(np.float32)
        g[: 2048] = (1e-18 * rng.standard_normal(2048)).astype(np.float32)  # v subnormal
        g[2048: 2048 + 64] = 0.0
        return oracle.f32_to_bf16_rne(g) if gdt_ == "bf16" else g
    say(f"tiny second moments {pdt}/{gdt}")
    run_small(q, [4 * 2048 + 77], pdt, gdt, steps=3, seed=11, grads=grads)


@pytest.mark.parametrize("gdt", ["bf16", "f32"])
@pytest.mark.parametrize("hp", [HP,
                                dict(lr=5e-2, beta1=0.5, beta2=0.75, eps=1e-6),
                                dict(lr=1e-4, beta1=0.95, beta2=0.9999, eps=0.0),
                                dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-40),
                                dict(lr=4e6, beta1=0.9, beta2=0.999, eps=1e-8)])
def test_bf16_params_short_path(q, hp, gdt):
    """bf16 parameters over 2^19 + 333 elements: the kernel's short path for bf16
    results (hardware square root and reciprocal behind an error screen) must give
    the oracle's bf16 bits everywhere.  lr = 5e-2 puts many updates next to the
    parameter's own size, so many slices fail the screen and take the correctly
    rounded path; a subnormal eps and a step size above 2^20 switch the screen off."""
    say(f"bf16 short path {hp} grads {gdt}")
    run_small(q, [2 ** 19 + 333], "bf16", gdt, steps=3, seed=12, hp=hp)


def step_from_state(q, p, g, cm, cv, am, av, pdt, gdt, step, hp):
    """One kernel step from the given host state against the oracle's, every element."""
    dp, dg = to_dev(p, pdt), to_dev(g, gdt)
    ds = [torch.from_numpy(x.copy()).cuda() for x in (cm, cv, am, av)]
    q.qopt_adam8bit_step([(dp, dg, *ds)], step=step, **hp)
    ref = oracle.adam8bit_step(p, g, cm, cv, am, av, step=step, param_dtype=pdt,
                               grad_dtype=gdt, **hp)
    torch.cuda.synchronize()
    what = f"({pdt}/{gdt}, step {step}, {hp})"
    assert_state([t.cpu().numpy() for t in ds], list(ref[1:]), what)
    assert_params(to_host(dp, pdt), ref[0], pdt, hp["lr"], what)
    return ref[0]


@pytest.mark.parametrize("gdt", ["bf16", "f32"])
def test_bf16_quotient_overflow(q, gdt):
    """Large first moments over small second moments with eps = 0: m / denominator
    overflows binary32 for part of the elements (the sequence's parameter becomes
    infinite) while step_size * m / denominator does not.  The bf16 short path never
    forms that quotient; its bound on |t| must send those slices to the sequence."""
    rng = np.random.default_rng(31)
    n = 16 * 2048
    p = oracle.f32_to_bf16_rne(rng.normal(0, 1.0, n).astype(np.float32))
    g = np.zeros(n, np.float32)
    g = oracle.f32_to_bf16_rne(g) if gdt == "bf16" else g
    cm = rng.integers(0, 256, n).astype(np.uint8)
    cv = rng.integers(1, 256, n).astype(np.uint8)
    am = np.full(16, 1e30, np.float32)
    av = (10.0 ** rng.uniform(-22, -16, 16)).astype(np.float32)
    say(f"bf16 quotient overflow grads {gdt}")
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        ref = step_from_state(q, p, g, cm, cv, am, av, "bf16", gdt, 1000,
                              dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=0.0))
    inf = np.count_nonzero((ref & 0x7FFF) == 0x7F80)
    assert 100 < inf < n - 100


@pytest.mark.parametrize("eps", [1e-30, 1e-8, 0.0])
def test_bf16_subnormal_second_moments(q, eps):
    """Second moments spread over the subnormals and the smallest normals.  The
    hardware square root flushes subnormal inputs to zero: with eps = 1e-30 the
    kernel checks every slice for them, with eps = 1e-8 (large enough) and eps = 0
    (denominator 0, t rejected by its bound) it does not, and all three must give the
    oracle's bits."""
    rng = np.random.default_rng(33)
    n = 16 * 2048 + 5
    nb = -(-n // BLOCK)
    p = oracle.f32_to_bf16_rne(rng.normal(0, 0.02, n).astype(np.float32))
    g = (rng.choice([-1.0, 1.0], n) * 10.0 ** rng.uniform(-24, -18, n)).astype(np.float32)
    g = oracle.f32_to_bf16_rne(g)
    cm = rng.integers(0, 256, n).astype(np.uint8)
    cv = rng.integers(0, 256, n).astype(np.uint8)
    am = (10.0 ** rng.uniform(-9, -6, nb)).astype(np.float32)
    av = (10.0 ** rng.uniform(-44, -36, nb)).astype(np.float32)
    say(f"bf16 subnormal second moments eps={eps}")
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        step_from_state(q, p, g, cm, cv, am, av, "bf16", "bf16", 3,
                        dict(lr=5e-2, beta1=0.5, beta2=0.75, eps=eps))


@pytest.mark.parametrize("pdt,gdt", [("f32", "bf16"), ("bf16", "bf16"), ("f32", "f32")])
def test_non_finite_gradients_follow_the_oracle(q, pdt, gdt):
    """Non-finite gradients are outside the method's contract; the step still follows
    the oracle's reading of them, code for code and block maximum for block maximum,
    in the poisoned blocks too: a NaN moment makes its block's maximum NaN and the
    block is stored as zero; an infinite one gives a reciprocal of 0, so the block's
    finite moments encode as 0 and the infinite one as the top code, and the next
    step decodes that block to NaN (0 times inf).  Parameters of the other blocks
    match as usual, and the poisoned blocks' parameters are NaN exactly where the
    oracle's are, equal elsewhere."""
    n = 6 * 2048 + 100
    rng = np.random.default_rng(41)
    p = host_params(n, pdt, rng)
    hs = host_state(n)
    dp, ds = to_dev(p, pdt), dev_state(n)
    bad_blocks = (1, 4)
    keep = np.ones(n, bool)
    for b in bad_blocks:
        keep[b * BLOCK:(b + 1) * BLOCK] = False
    say(f"non-finite gradients {pdt}/{gdt}")
    for step in range(1, 4):
        g = rng.normal(0, 1e-3, n).astype(np.float32)
        g[1 * BLOCK + 7] = np.nan
        g[1 * BLOCK + 300] = np.inf
        g[4 * BLOCK + 2047] = -np.inf if step == 1 else g[4 * BLOCK + 2047]
        g = oracle.f32_to_bf16_rne(g) if gdt == "bf16" else g
        q.qopt_adam8bit_step([(dp, to_dev(g, gdt), *ds)], step=step, **HP)
        with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
            out = oracle.adam8bit_step(p, g, *hs, step=step, param_dtype=pdt, grad_dtype=gdt, **HP)
        p, hs = out[0], list(out[1:])
        torch.cuda.synchronize()
        got = [t.cpu().numpy() for t in ds]
        what = f"(step {step}, {pdt}/{gdt})"
        assert_state(got, hs, what)
        gp = to_host(dp, pdt)
        assert_params(gp[keep], p[keep], pdt, HP["lr"], what)
        gp32 = oracle.bf16_to_f32(gp) if pdt == "bf16" else gp
        p32 = oracle.bf16_to_f32(p) if pdt == "bf16" else p
        nan_ref = np.isnan(p32[~keep])
        assert np.array_equal(np.isnan(gp32[~keep]), nan_ref), what
        assert_params(gp[~keep][~nan_ref], p[~keep][~nan_ref], pdt, HP["lr"], what)
    # after step 1 block 4 held -inf as its m maximum and inf as its v maximum
    # (checked through the oracle above); by step 3 both poisoned blocks are NaN
    assert hs[2][1] == 0 and hs[3][1] == 0


@pytest.mark.parametrize("pdt,gdt", [("f32", "f32"), ("f32", "bf16"), ("bf16", "f32"),
                                     ("bf16", "bf16")])
def test_traffic_probe_keeps_every_buffer(q, pdt, gdt):
    """The measurement aid moves the step's bytes and writes back what it read: after
    it, parameters, gradients, codes and block maxima are bit for bit unchanged (tails
    and misaligned views are skipped by it, full blocks rewritten)."""
    sizes = [5 * 2048, 2048 + 3, 7, 3 * 2048]
    rng = np.random.default_rng(51)
    ts = []
    for n in sizes:
        nb = -(-n // BLOCK)
        ts.append((to_dev(host_params(n, pdt, rng), pdt), to_dev(host_grads(n, gdt, rng), gdt),
                   torch.from_numpy(rng.integers(0, 256, n).astype(np.uint8)).cuda(),
                   torch.from_numpy(rng.integers(0, 256, n).astype(np.uint8)).cuda(),
                   torch.from_numpy(rng.random(nb).astype(np.float32)).cuda(),
                   torch.from_numpy(rng.random(nb).astype(np.float32)).cuda()))
    before = [[t.clone() for t in tup] for tup in ts]
    say(f"traffic probe {pdt}/{gdt}")
    for _ in range(3):
        q.qopt_adam8bit_traffic_probe(ts)
    torch.cuda.synchronize()
    for tup, ref in zip(ts, before):
        for a, b in zip(tup, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_pattern_probes_keep_every_buffer(q):
    """Every bytes-only pattern of the ceiling study writes back what it read: after
    each, parameters, gradients and codes are bit for bit unchanged (a ragged last
    burst of the burst patterns is left out, not corrupted)."""
    nblk = 3 * 8 * 4 * 256 + 5       # several runs of every walk, and a partial burst
    n = nblk * BLOCK
    rng = np.random.default_rng(61)
    p = torch.from_numpy(rng.normal(0, 0.02, n).astype(np.float32)).cuda()
    g = torch.from_numpy(rng.normal(0, 1e-3, n).astype(np.float32)).cuda().bfloat16()
    cm = torch.from_numpy(rng.integers(0, 256, n, dtype=np.uint8)).cuda()
    cv = torch.from_numpy(rng.integers(0, 256, n, dtype=np.uint8)).cuda()
    ref = [t.clone() for t in (p, g, cm, cv)]
    names = q.qopt_pattern_probe_names()
    for i, name in enumerate(names):
        say(f"pattern probe {i}: {name}")
        q.qopt_pattern_probe(i, p, g, cm, cv)
        torch.cuda.synchronize()
        for a, b in zip((p, g, cm, cv), ref):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), name


@pytest.mark.parametrize("pdt,gdt", [("f32", "f32"), ("f32", "bf16"), ("bf16", "f32"),
                                     ("bf16", "bf16")])
def test_random_hyperparameters(q, pdt, gdt):
    """Thirty-two seeded hyper-parameter draws per dtype pair.  The draws cover:
    - lr from 1e-5 to 1e-1;
    - beta1 in [0, 0.99) and beta2 in [0.5, 0.9999);
    - eps among 0, a subnormal, 1e-30, 1e-12, 1e-8 and 1e-6;
    - steps 1 to 1000.

    Every bf16 screen mode and fallback runs.  Each draw compares every element
    after two consecutive steps."""
    rng = np.random.default_rng(61 + sum(map(ord, pdt + gdt)))
    for d in range(32):
        hp = dict(lr=float(10.0 ** rng.uniform(-5, -1)), beta1=float(rng.uniform(0.0, 0.99)),
                  beta2=float(1.0 - 10.0 ** rng.uniform(-4, np.log10(0.5))),
                  eps=float(rng.choice([0.0, 1e-40, 1e-30, 1e-12, 1e-8, 1e-6])))
        step0 = int(rng.choice([0, 1, 9, 999]))
        sizes = [2 * 2048 + 77, 4096]
        hp_p = [host_params(n, pdt, rng) for n in sizes]
        hs = [host_state(n) for n in sizes]
        dp = [to_dev(p, pdt) for p in hp_p]
        ds = [dev_state(n) for n in sizes]
        say(f"draw {d}: {hp} from step {step0 + 1} {pdt}/{gdt}")
        for step in (step0 + 1, step0 + 2):
            hg = [host_grads(n, gdt, rng, scale=float(10.0 ** rng.uniform(-6, 0))) for n in sizes]
            q.qopt_adam8bit_step([(dp[i], to_dev(hg[i], gdt), *ds[i]) for i in range(len(sizes))],
                                 step=step, **hp)
            for i in range(len(sizes)):
                out = oracle.adam8bit_step(hp_p[i], hg[i], *hs[i], step=step, param_dtype=pdt,
                                           grad_dtype=gdt, **hp)
                hp_p[i], hs[i] = out[0], list(out[1:])
            torch.cuda.synchronize()
            for i, n in enumerate(sizes):
                what = f"(draw {d}, tensor {i}, step {step}, {hp}, {pdt}/{gdt})"
                assert_state([t.cpu().numpy() for t in ds[i]], hs[i], what)
                assert_params(to_host(dp[i], pdt), hp_p[i], pdt, hp["lr"], what)


def test_late_step_and_zero_blocks(q):
    """A large step number, and blocks whose gradient and state are zero."""
    n = 4 * 2048
    p0 = np.random.default_rng(7).normal(0, 0.02, n).astype(np.float32)
    g = np.zeros(n, np.float32)
    g[2048:4096] = 1e-3
    p = torch.from_numpy(p0.copy()).cuda()
    st = dev_state(n)
    q.qopt_adam8bit_step([(p, torch.from_numpy(g).cuda(), *st)], step=1_000_003, **HP)
    ref = oracle.adam8bit_step(p0, g, *host_state(n), step=1_000_003, **HP)
    torch.cuda.synchronize()
    assert_state([t.cpu().numpy() for t in st], ref[1:])
    assert_params(p.cpu().numpy(), ref[0], "f32", HP["lr"])
    assert np.array_equal(p.cpu().numpy()[:2048], p0[:2048])


def test_optimizer_class_and_resume(q):
    """Adam8bit on two parameters; a state_dict round trip resumes bit-exactly."""
    torch.manual_seed(0)
    w = torch.nn.Parameter(torch.randn(3000, device="cuda") * 0.02)
    b = torch.nn.Parameter((torch.randn(2048 * 2 + 3, device="cuda") * 0.02).bfloat16())
    opt = q.Adam8bit([w, b], lr=1e-3)
    ref_w = [w.detach().cpu().numpy().copy(), *host_state(w.numel())]
    ref_b = [to_host(b.detach(), "bf16").copy(), *host_state(b.numel())]
    rng = np.random.default_rng(8)
    saved = None
    for step in range(1, 7):
        gw = rng.normal(0, 1e-3, w.numel()).astype(np.float32)
        gb = oracle.f32_to_bf16_rne(rng.normal(0, 1e-3, b.numel()).astype(np.float32))
        w.grad = torch.from_numpy(gw).cuda()
        b.grad = to_dev(gb, "bf16")
        opt.step()
        ref_w = list(oracle.adam8bit_step(ref_w[0], gw, *ref_w[1:], step=step, **HP))
        ref_b = list(oracle.adam8bit_step(ref_b[0], gb, *ref_b[1:], step=step,
                                          param_dtype="bf16", grad_dtype="bf16", **HP))
        if step == 3:
            saved = (copy.deepcopy(opt.state_dict()), w.detach().clone(), b.detach().clone())
    torch.cuda.synchronize()
    assert_params(w.detach().cpu().numpy(), ref_w[0], "f32", 1e-3)
    assert_params(to_host(b.detach(), "bf16"), ref_b[0], "bf16", 1e-3)
    st = opt.state[w]
    assert_state([st[k].cpu().numpy() for k in ("m_codes", "v_codes", "m_absmax", "v_absmax")],
                 ref_w[1:])
    final_w, final_b = w.detach().clone(), b.detach().clone()
    # resume from step 3 in a fresh optimizer and replay steps 4..6
    with torch.no_grad():
        w.copy_(saved[1])
        b.copy_(saved[2])
    opt2 = q.Adam8bit([w, b], lr=1e-3)
    opt2.load_state_dict(saved[0])
    assert opt2.state[b]["m_absmax"].dtype == torch.float32
    rng = np.random.default_rng(8)
    for step in range(1, 7):
        gw = rng.normal(0, 1e-3, w.numel()).astype(np.float32)
        gb = oracle.f32_to_bf16_rne(rng.normal(0, 1e-3, b.numel()).astype(np.float32))
        if step <= 3:
            continue
        w.grad = torch.from_numpy(gw).cuda()
        b.grad = to_dev(gb, "bf16")
        opt2.step()
    torch.cuda.synchronize()
    assert torch.equal(w.detach(), final_w) and torch.equal(b.detach(), final_b)


def _busy(stream, n=4096, reps=12):
    """Queue several milliseconds of matrix products on ``stream``."""
    with torch.cuda.stream(stream):
        a = torch.full((n, n), 1.0 / n, device="cuda")  # a @ a == a
        for _ in range(reps):
            a = a @ a
    return a


def test_step_runs_on_the_callers_stream(q):
    """The step goes on the caller's current stream: on a side stream (default
    priority) queued behind long matrix products and the copy that fills the
    gradients, it must see those gradients, and its results must equal the oracle's.
    A step queued anywhere else would read the zero gradients the copy overwrites."""
    rng = np.random.default_rng(2024)
    sizes = [3 * BLOCK + 5, 40 * BLOCK]
    pdt, gdt = "f32", "bf16"
    hp_p = [host_params(n, pdt, rng) for n in sizes]
    hg = [host_grads(n, gdt, rng) for n in sizes]
    dp = [to_dev(p, pdt) for p in hp_p]
    ds = [dev_state(n) for n in sizes]
    src = [to_dev(g, gdt) for g in hg]
    dg = [torch.zeros_like(t) for t in src]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    say(f"side stream step sizes={sizes}")
    _busy(side)
    with torch.cuda.stream(side):
        for d, g in zip(dg, src):
            d.copy_(g)
        q.qopt_adam8bit_step([(dp[i], dg[i], *ds[i]) for i in range(len(sizes))], step=1, **HP)
    side.synchronize()
    for i, n in enumerate(sizes):
        hs = host_state(n)
        out = oracle.adam8bit_step(hp_p[i], hg[i], *hs, step=1, param_dtype=pdt, grad_dtype=gdt,
                                   **HP)
        what = f"(tensor {i}, n={n}, side stream)"
        assert_state([t.cpu().numpy() for t in ds[i]], list(out[1:]), what)
        assert_params(to_host(dp[i], pdt), out[0], pdt, HP["lr"], what)


def test_bf16_step_runs_on_the_callers_stream(q, tmp_path):
    """bf16 parameters with two launches (2^18 + 3000 blocks), which the step spreads
    over the caller's stream and a second stream of the library's: on a side stream
    queued behind long matrix products and the copy that fills the gradients, both
    launches must see those gradients (the second stream waits for the caller's), and
    sampled blocks on both sides of the launch split must match the oracle."""
    nblk = (1 << 18) + 3000
    n = nblk * BLOCK
    P = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    workloads.fill_normal_(P, 0.02, 21)
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    workloads.fill_normal_(src, 1e-3, 22)
    G = torch.zeros_like(src)
    st = dev_state(n)
    assert q.qopt_adam8bit_launch_count([(P, G, *st)]) == 2
    half = -(-nblk // 2)
    sample = workloads.sample_blocks(nblk, 300, 23, must=[half - 1, half])
    sidx = torch.from_numpy(sample).cuda()

    def gather(flat, dtype):
        return to_host(flat.view(-1, BLOCK)[sidx].reshape(-1), dtype)

    inputs = {"p0": gather(P, "bf16"), "g1": gather(src, "bf16")}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    say(f"side stream bf16 step, {nblk} blocks")
    _busy(side)
    with torch.cuda.stream(side):
        G.copy_(src)
        q.qopt_adam8bit_step([(P, G, *st)], step=1, **HP)
    side.synchronize()
    got = [gather(st[0], "u8"), gather(st[1], "u8"), st[2][sidx].cpu().numpy(), st[3][sidx].cpu().numpy()]
    gp = gather(P, "bf16")
    ref = run_oracle_blocks(inputs, dict(HP, steps=1, pdt="bf16", gdt="bf16"), sample.size, str(tmp_path))
    what = f"({sample.size} sampled blocks, side stream)"
    assert_state(got, [ref["cm"], ref["cv"], ref["am"], ref["av"]], what)
    assert_params(gp, ref["p"], "bf16", HP["lr"], what)
    del P, src, G, st
    torch.cuda.empty_cache()


def test_steps_from_two_threads_on_two_streams(q):
    """Two host threads step two disjoint tensor sets at once, each on its own stream
    (default priority): the library keeps no per-call state, so both match the oracle."""
    import threading
    sizes = {"a": [5 * BLOCK + 3, 17 * BLOCK], "b": [BLOCK - 1, 23 * BLOCK + 100]}
    pdt, gdt = "f32", "bf16"
    rng = np.random.default_rng(4242)
    hp_p = {k: [host_params(n, pdt, rng) for n in v] for k, v in sizes.items()}
    hg = {k: [[host_grads(n, gdt, rng) for n in v] for _ in range(3)] for k, v in sizes.items()}
    dp = {k: [to_dev(p, pdt) for p in hp_p[k]] for k in sizes}
    ds = {k: [dev_state(n) for n in v] for k, v in sizes.items()}
    dg = {k: [[to_dev(g, gdt) for g in step] for step in hg[k]] for k in sizes}
    torch.cuda.synchronize()
    errors = []

    def run(k):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for step in range(1, 4):
                    q.qopt_adam8bit_step([(dp[k][i], dg[k][step - 1][i], *ds[k][i])
                                          for i in range(len(sizes[k]))], step=step, **HP)
            stream.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    say(f"two threads, sizes={sizes}")
    threads = [threading.Thread(target=run, args=(k,)) for k in sizes]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for k, v in sizes.items():
        for i, n in enumerate(v):
            p, st = hp_p[k][i], host_state(n)
            for step in range(1, 4):
                out = oracle.adam8bit_step(p, hg[k][step - 1][i], *st, step=step, param_dtype=pdt,
                                           grad_dtype=gdt, **HP)
                p, st = out[0], list(out[1:])
            what = f"(set {k}, tensor {i}, n={n})"
            assert_state([t.cpu().numpy() for t in ds[k][i]], st, what)
            assert_params(to_host(dp[k][i], pdt), p, pdt, HP["lr"], what)


def test_optimizer_per_parameter_steps(q):
    """A parameter without a gradient skips the step and keeps its own step count
    (as torch.optim.Adam does); the parameters then fall into separate launches per
    (device, dtypes, step), each following the oracle with its own count, and each
    batch's launch descriptors are built once and reused."""
    torch.manual_seed(1)
    a = torch.nn.Parameter(torch.randn(5000, device="cuda") * 0.02)
    b = torch.nn.Parameter(torch.randn(2048 + 9, device="cuda") * 0.02)
    c = torch.nn.Parameter((torch.randn(4097, device="cuda") * 0.02).bfloat16())
    opt = q.Adam8bit([a, b, c], lr=1e-3)
    refs = {"a": [a.detach().cpu().numpy().copy(), *host_state(a.numel())],
            "b": [b.detach().cpu().numpy().copy(), *host_state(b.numel())],
            "c": [to_host(c.detach(), "bf16").copy(), *host_state(c.numel())]}
    steps = {"a": 0, "b": 0, "c": 0}
    params = {"a": a, "b": b, "c": c}
    rng = np.random.default_rng(9)
    plan = [("a", "b", "c"), ("a",), ("a", "b", "c"), ("a", "c"), ("a", "b", "c")]
    for it, live in enumerate(plan):
        for name, p in params.items():
            p.grad = None
        for name in live:
            p = params[name]
            g = rng.normal(0, 1e-3, p.numel()).astype(np.float32)
            dt = "bf16" if p.dtype == torch.bfloat16 else "f32"
            if dt == "bf16":
                g = oracle.f32_to_bf16_rne(g)
            p.grad = to_dev(g, dt)
            steps[name] += 1
            r = refs[name]
            refs[name] = list(oracle.adam8bit_step(r[0], g, *r[1:], step=steps[name],
                                                   param_dtype=dt, grad_dtype=dt, **HP))
        opt.step()
        torch.cuda.synchronize()
        for name, p in params.items():
            dt = "bf16" if p.dtype == torch.bfloat16 else "f32"
            what = f"({name}, iteration {it + 1}, step {steps[name]})"
            assert opt.state[p].get("step", 0) == steps[name], what
            assert_params(to_host(p.detach(), dt), refs[name][0], dt, 1e-3, what)
            if steps[name]:
                st = opt.state[p]
                assert_state([st[k].cpu().numpy()
                              for k in ("m_codes", "v_codes", "m_absmax", "v_absmax")],
                             refs[name][1:], what)
    # a steady batch reuses its cached launch descriptors
    for name, p in params.items():
        p.grad = torch.zeros_like(p)
    opt.step()
    cached = dict(opt._prepared)
    opt.step()
    assert opt._prepared.keys() == cached.keys()
    assert all(opt._prepared[k] is cached[k] for k in cached)


# ------------------------------------------------------- full-size, sampled


ORACLE_WORKERS = 8   # child processes running the oracle (numpy only)


def run_oracle_blocks(inputs, cfg, nblocks, tmpdir):
    """The oracle's trajectory of the gathered full blocks (``inputs``: p0 and the
    gradients of every step, blocks one after another), split over ORACLE_WORKERS
    child processes by block; returns the final parameters, codes and block maxima."""
    worker = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_blocks_worker.py")
    cuts = np.linspace(0, nblocks, ORACLE_WORKERS + 1).astype(np.int64)
    procs = []
    for w in range(ORACLE_WORKERS):
        a, b = int(cuts[w]) * BLOCK, int(cuts[w + 1]) * BLOCK
        if a == b:
            continue
        fin, fout = os.path.join(tmpdir, f"in{w}.npz"), os.path.join(tmpdir, f"out{w}.npz")
        np.savez(fin, cfg=np.array(json.dumps(cfg)), **{k: v[a:b] for k, v in inputs.items()})
        procs.append((fout, subprocess.Popen([sys.executable, worker, fin, fout])))
    outs = []
    for fout, pr in procs:
        assert pr.wait() == 0, "oracle worker failed"
        outs.append(np.load(fout))
    return {k: np.concatenate([o[k] for o in outs]) for k in ("p", "cm", "cv", "am", "av")}


def sampled_trajectory(q, shapes, pdt, gdt, steps, seed, grad_fill, tmp_path, sample_frac=0.01,
                       extra_blocks=()):
    """Run ``steps`` GPU steps over a full parameter set from zero state and follow at
    least ``sample_frac`` of its blocks in the oracle, which can step them on their
    own because blocks are independent: every tensor's first and last block, the
    blocks on either side of every launch split of the step's plan (launches cover
    equal runs of the flattened blocks), the extra blocks, and distinct blocks drawn
    uniformly.  The parameter set lies in flat buffers with every tensor starting on
    a block boundary and every block full, so a sampled block is one row of the
    buffers viewed as [blocks, 2048]."""
    dt_p, dt_g = DT[pdt], DT[gdt]
    offs = np.cumsum([0] + [n for _, n in shapes])
    assert all(n % BLOCK == 0 for _, n in shapes)
    total = int(offs[-1])
    nblk = total // BLOCK
    say(f"allocating {len(shapes)} tensors, {total} params ({pdt} params, {gdt} grads)")
    P = torch.empty(total, dtype=dt_p, device="cuda")
    G = torch.empty(total, dtype=dt_g, device="cuda")
    CM = torch.zeros(total, dtype=torch.uint8, device="cuda")
    CV = torch.zeros_like(CM)
    AM = torch.zeros(nblk, dtype=torch.float32, device="cuda")
    AV = torch.zeros_like(AM)
    workloads.fill_normal_(P, 0.02, seed)
    tensors = []
    for ti, (name, n) in enumerate(shapes):
        o, bo = int(offs[ti]), int(offs[ti]) // BLOCK
        tensors.append((P[o:o + n], G[o:o + n], CM[o:o + n], CV[o:o + n],
                        AM[bo:bo + n // BLOCK], AV[bo:bo + n // BLOCK]))
    nlaunch = q.qopt_adam8bit_launch_count(tensors)
    per_launch = -(-nblk // nlaunch)
    splits = [k * per_launch for k in range(1, nlaunch)]
    starts = offs[:-1] // BLOCK
    must = list(extra_blocks) + [int(b) for b in starts] + [int(b) - 1 for b in offs[1:] // BLOCK]
    must += [b for s in splits for b in (s - 1, s)]
    sample = workloads.sample_blocks(nblk, int(np.ceil(sample_frac * nblk)), seed, must=must)
    assert sample.size >= sample_frac * nblk and set(must) <= set(sample.tolist())
    say(f"{nlaunch} launches, {sample.size} sampled blocks of {nblk} "
        f"({100.0 * sample.size / nblk:.2f} %)")
    sidx = torch.from_numpy(sample).cuda()

    def gather(flat, dtype):
        return to_host(flat.view(-1, BLOCK)[sidx].reshape(-1), dtype)

    inputs = {"p0": gather(P, pdt)}
    for step in range(1, steps + 1):
        grad_fill(G, step)
        inputs[f"g{step}"] = gather(G, gdt)
        q.qopt_adam8bit_step(tensors, step=step, **HP)
        torch.cuda.synchronize()
        say(f"step {step} done")
    got = [gather(CM, "u8"), gather(CV, "u8"), AM[sidx].cpu().numpy(), AV[sidx].cpu().numpy()]
    gp = gather(P, pdt)
    del tensors, P, G, CM, CV, AM, AV
    torch.cuda.empty_cache()
    cfg = dict(HP, steps=steps, pdt=pdt, gdt=gdt)
    ref = run_oracle_blocks(inputs, cfg, sample.size, str(tmp_path))
    assert_state(got, [ref["cm"], ref["cv"], ref["am"], ref["av"]], f"({sample.size} sampled blocks)")
    assert_params(gp, ref["p"], pdt, HP["lr"], f"({sample.size} sampled blocks)")


def test_bf16_steps_from_two_threads_on_two_streams(q, tmp_path):
    """bf16 parameters spread a step's launches over the caller's stream and a second
    stream of the library's: two host threads, each stepping its own tensor of
    2^18 + 3000 blocks (two launches) on its own stream, twice, while the other does
    the same.  Sampled blocks (both sides of the launch split among them) must match
    the oracle."""
    import threading
    nblk = (1 << 18) + 3000
    n = nblk * BLOCK
    sets = {}
    for k, seed in (("a", 11), ("b", 12)):
        P = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        workloads.fill_normal_(P, 0.02, seed)
        G = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        for i, g in enumerate(G):
            workloads.fill_normal_(g, 1e-3, seed * 10 + i)
        st = dev_state(n)
        sets[k] = (P, G, st)
    nlaunch = q.qopt_adam8bit_launch_count([(sets["a"][0], sets["a"][1][0], *sets["a"][2])])
    assert nlaunch == 2
    half = -(-nblk // 2)
    sample = workloads.sample_blocks(nblk, 300, 5, must=[half - 1, half])
    sidx = torch.from_numpy(sample).cuda()

    def gather(flat, dtype):
        return to_host(flat.view(-1, BLOCK)[sidx].reshape(-1), dtype)

    inputs = {k: {"p0": gather(P, "bf16"), "g1": gather(G[0], "bf16"), "g2": gather(G[1], "bf16")}
              for k, (P, G, st) in sets.items()}
    torch.cuda.synchronize()
    errors = []

    def run(k):
        try:
            P, G, st = sets[k]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for step in (1, 2):
                    q.qopt_adam8bit_step([(P, G[step - 1], *st)], step=step, **HP)
            stream.synchronize()
        except Exception as e:  # reported below, in the main thread
            errors.append(e)

    say(f"two threads, bf16 params, {nblk} blocks each, {nlaunch} launches per step")
    threads = [threading.Thread(target=run, args=(k,)) for k in sets]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    cfg = dict(HP, steps=2, pdt="bf16", gdt="bf16")
    for k, (P, G, st) in sets.items():
        got = [gather(st[0], "u8"), gather(st[1], "u8"), st[2][sidx].cpu().numpy(), st[3][sidx].cpu().numpy()]
        gp = gather(P, "bf16")
        sub = tmp_path / k
        sub.mkdir()
        ref = run_oracle_blocks(inputs[k], cfg, sample.size, str(sub))
        what = f"(set {k}, {sample.size} sampled blocks)"
        assert_state(got, [ref["cm"], ref["cv"], ref["am"], ref["av"]], what)
        assert_params(gp, ref["p"], "bf16", HP["lr"], what)
    del sets
    torch.cuda.empty_cache()


def _dense_grads(std, seed, outlier_frac=0.0, outlier_scale=1.0):
    def fill(G, step):
        workloads.fill_normal_(G, std, seed * 1000 + step)
        if outlier_frac:
            workloads.scale_random_entries_(G, outlier_frac, outlier_scale, seed * 1000 + step)
    return fill


def test_fp32_step_past_32_bit_element_offsets(q, tmp_path):
    """One fp32-parameter tensor of 2^32 + 5 * 2048 elements with bf16 gradients, so
    that element offsets pass 2^31 and 2^32 inside one tensor (and inside one
    launch): the blocks on either side of both boundaries and a sample of the rest
    through two steps, against the oracle."""
    b31, b32 = (1 << 31) // BLOCK, (1 << 32) // BLOCK
    sampled_trajectory(q, [("huge", (1 << 32) + 5 * BLOCK)], "f32", "bf16", steps=2, seed=6,
                       grad_fill=_dense_grads(1e-3, 6, 1e-4, 1000.0), tmp_path=tmp_path,
                       sample_frac=0.0005, extra_blocks=[b31 - 1, b31, b32 - 1, b32])


@pytest.mark.parametrize("pdt,gdt", [("f32", "bf16"), ("bf16", "bf16"), ("f32", "f32")])
def test_every_block_of_long_launches(q, pdt, gdt, tmp_path):
    """Launches long enough for every wave to take several whole runs of consecutive
    blocks, with remainders that do not fill a round, and a second tensor whose
    launch is short: every block (the runs, the single blocks after them, the short
    launch's) is followed through two steps in the oracle, so a block the walk skips
    or takes twice cannot pass."""
    shapes = [("long", (3 * 8192 + 777) * BLOCK), ("short", 301 * BLOCK)]
    sampled_trajectory(q, shapes, pdt, gdt, steps=2, seed=23, grad_fill=_dense_grads(1e-3, 23),
                       tmp_path=tmp_path, sample_frac=1.0)


def test_gpt1p3b_sampled(q, tmp_path):
    sampled_trajectory(q, workloads.gpt1p3b_shapes(), "f32", "bf16", steps=6, seed=2,
                       grad_fill=_dense_grads(1e-3, 2), tmp_path=tmp_path)


def test_llama7b_sampled(q, tmp_path):
    sampled_trajectory(q, workloads.llama7b_shapes(), "f32", "bf16", steps=6, seed=3,
                       grad_fill=_dense_grads(1e-3, 3, 1e-4, 1000.0), tmp_path=tmp_path)


def test_flat20b_sampled(q, tmp_path):
    rows, dim = workloads.FLAT20B_EMBED_ROWS, workloads.FLAT20B_EMBED_DIM
    emb = rows * dim

    def fill(G, step):
        workloads.fill_normal_(G, 5e-4, 4000 + step)
        mask = workloads.sparse_rows_mask(rows, workloads.FLAT20B_ACTIVE_ROWS, 4000 + step,
                                          G.device)
        G[:emb].view(rows, dim)[~mask] = 0

    extra = [emb // BLOCK - 1, emb // BLOCK, 7, 1000]
    sampled_trajectory(q, [("flat", workloads.FLAT20B_N)], "bf16", "bf16", steps=3, seed=4,
                       grad_fill=fill, tmp_path=tmp_path, extra_blocks=extra)
