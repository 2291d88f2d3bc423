"""GPU parity of the block-wise quantize / dequantize kernels against the oracle.

Codes and absmax must be bit-exact; dequantized values too (one binary32 multiply
on both sides).  Sizes span several blocks and ragged tails; the full 2^28-value
Student-t workload is checked on sampled blocks plus whole-size properties; every
binary32 in [0, 1] is swept through both codebooks.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu
KINDS = [oracle.SIGNED, oracle.UNSIGNED]
SIZES = [1, 7, 2047, 2048, 2049, 50257, 3 * 2048 + 5, 40 * 2048 + 1234]


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_wise_bit_adam8bit_amd as q
    torch.cuda.set_device(0)
    return q


def _check_codec(q, x, kind, xd=None, codes=None, absmax=None):
    xd = torch.from_numpy(x).cuda() if xd is None else xd
    c, a = q.qopt_quantize_blockwise(xd, kind, codes=codes, absmax=absmax)
    y = q.qopt_dequantize_blockwise(c, a, kind)
    c_ref, a_ref = oracle.quantize_blockwise(x, kind)
    y_ref = oracle.dequantize_blockwise(c_ref, a_ref, kind)
    torch.cuda.synchronize()
    c_got = c.cpu().numpy()
    bad = np.nonzero(c_got != c_ref)[0]
    assert bad.size == 0, f"{bad.size} codes differ, first at {bad[:5]}: {c_got[bad[:5]]} vs {c_ref[bad[:5]]}"
    assert np.array_equal(a.cpu().numpy().view(np.uint32), a_ref.view(np.uint32))
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n", SIZES)
def test_codec_matches_oracle(q, kind, n):
    say(f"codec kind={kind} n={n}")
    x = workloads.student_t3_host(n, seed=n)
    _check_codec(q, x, kind)
    if kind == oracle.UNSIGNED:
        _check_codec(q, np.abs(x), kind)


@pytest.mark.parametrize("kind", KINDS)
def test_block_max_at_every_position(q, kind):
    """Block b's unique largest magnitude sits at element b of the block, so over
    2048 blocks the maximum is held once by every lane in every slice; the block
    maxima (a reduction across the wave) and all codes must still be exact."""
    say(f"block max at every position, kind={kind}")
    rng = np.random.default_rng(11)
    x = rng.uniform(-0.5, 0.5, (workloads.BLOCK, workloads.BLOCK)).astype(np.float32)
    b = np.arange(workloads.BLOCK)
    x[b, b] = (np.where(b % 2 == 0, 1.0, -1.0) * (1.0 + b / 4096.0)).astype(np.float32)
    x = x.reshape(-1)
    if kind == oracle.UNSIGNED:
        x = np.abs(x)
    _check_codec(q, x, kind)


def test_codec_runs_on_the_callers_stream(q):
    """Quantize and dequantize go on the caller's current stream: on a side stream
    (default priority) queued behind long matrix products and the copy that fills
    their input, they must see that input, and their outputs must equal the oracle's."""
    kind = oracle.SIGNED
    x = workloads.student_t3_host(5 * 2048 + 77, seed=31)
    src = torch.from_numpy(x).cuda()
    xd = torch.zeros_like(src)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    say(f"side stream codec n={x.size}")
    with torch.cuda.stream(side):
        a = torch.full((4096, 4096), 1.0 / 4096, device="cuda")  # a @ a == a
        for _ in range(12):
            a = a @ a
        xd.copy_(src)
        c, m = q.qopt_quantize_blockwise(xd, kind)
        y = q.qopt_dequantize_blockwise(c, m, kind)
    side.synchronize()
    c_ref, a_ref = oracle.quantize_blockwise(x, kind)
    y_ref = oracle.dequantize_blockwise(c_ref, a_ref, kind)
    assert np.array_equal(c.cpu().numpy(), c_ref)
    assert np.array_equal(m.cpu().numpy().view(np.uint32), a_ref.view(np.uint32))
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))


@pytest.mark.parametrize("kind", KINDS)
def test_codec_misaligned_views(q, kind):
    """Views at element offsets that break 16-byte (x) and 4-byte (codes) alignment
    take the element-wise path and still match."""
    n = 5 * 2048 + 99
    x = workloads.student_t3_host(n, seed=5)
    buf = torch.zeros(n + 3, dtype=torch.float32, device="cuda")
    buf[1:n + 1] = torch.from_numpy(x).cuda()
    cbuf = torch.zeros(n + 3, dtype=torch.uint8, device="cuda")
    say(f"codec misaligned kind={kind}")
    _check_codec(q, x, kind, xd=buf[1:n + 1], codes=cbuf[3:n + 3])


@pytest.mark.parametrize("kind", KINDS)
def test_codec_special_blocks(q, kind):
    """Zero, subnormal, constant, single-outlier, signed-zero and threshold blocks."""
    B = 2048
    T = oracle.code_transitions(kind)
    mags = oracle.magnitudes_f32(kind)
    blocks = [np.zeros(B, np.float32),
              np.full(B, 1e-40, np.float32),
              np.full(B, -3.5, np.float32),
              np.full(B, 2.0 ** -126, np.float32)]
    out = np.random.default_rng(1).normal(0, 1e-3, B).astype(np.float32)
    out[77] = 1e3
    blocks.append(out)
    sz = np.zeros(B, np.float32)
    sz[::2] = -0.0
    sz[5] = -1e-9
    sz[6] = 1.0
    blocks.append(sz)
    # values on and next to every decision threshold and table value, absmax 1
    adv = np.concatenate([T, np.nextafter(T, np.float32(0)), np.nextafter(T, np.float32(2)),
                          mags, (mags[:-1] + mags[1:]) / 2]).astype(np.float32)
    adv = np.concatenate([[1.0], adv, -adv if kind == oracle.SIGNED else adv]).astype(np.float32)
    adv = np.resize(adv, (-(-adv.size // B)) * B)
    adv[::B] = 1.0
    blocks.append(adv)
    x = np.concatenate(blocks).astype(np.float32)
    say(f"codec special blocks kind={kind} n={x.size}")
    _check_codec(q, x, kind)


@pytest.mark.parametrize("kind", KINDS)
def test_codec_non_finite_blocks(q, kind):
    """Blocks holding NaN or infinite values (outside the method's contract) still
    match the oracle code for code: a NaN anywhere makes the block's maximum NaN, so
    it is stored as absmax 0 with every code 0; an infinite maximum gives a reciprocal
    of 0, so finite elements encode as 0 (with their sign) and infinite ones as the
    top code.  Neighbouring blocks are untouched (block independence)."""
    B = 2048
    rng = np.random.default_rng(21)
    base = workloads.student_t3_host(9 * B + 100, seed=21)
    x = base.copy()
    x[1 * B + 5] = np.nan                       # one NaN
    x[2 * B + 9] = np.inf                       # one +inf
    x[3 * B + 2047] = -np.inf                   # one -inf, last lane of the last slice
    x[4 * B: 5 * B] = np.nan                    # all NaN
    x[5 * B + 3] = np.inf                       # NaN and inf together
    x[5 * B + 4] = np.nan
    x[6 * B: 7 * B] = -np.inf                   # all -inf
    x[7 * B + rng.integers(0, B, 40)] = np.inf  # many +inf
    x[9 * B + 50] = np.nan                      # in the short tail block
    if kind == oracle.UNSIGNED:
        x = np.abs(x)
    say(f"codec non-finite blocks kind={kind}")
    with np.errstate(invalid="ignore"):
        c_ref, a_ref = oracle.quantize_blockwise(x, kind)
    c, a = q.qopt_quantize_blockwise(torch.from_numpy(x).cuda(), kind)
    torch.cuda.synchronize()
    got_c, got_a = c.cpu().numpy(), a.cpu().numpy()
    bad = np.nonzero(got_c != c_ref)[0]
    assert bad.size == 0, f"{bad.size} codes differ, first at {bad[:5]}"
    assert np.array_equal(got_a.view(np.uint32), a_ref.view(np.uint32))
    # the oracle's reading, restated: NaN blocks zero, infinite blocks keep inf
    assert a_ref[1] == 0 and a_ref[4] == 0 and a_ref[5] == 0 and a_ref[9] == 0
    assert not c_ref[4 * B: 6 * B].any()
    assert np.isinf(a_ref[2]) and np.isinf(a_ref[7]) and np.isfinite(a_ref[8])


@pytest.mark.parametrize("kind", KINDS)
def test_exhaustive_unit_interval(q, kind):
    """Every binary32 in [0, 1] (and, signed, its negation) is quantized in blocks
    whose absmax is exactly 1.0, so the kernel encodes the value itself.  The codes
    of the ordered sweep must step by one exactly at the oracle's transition points
    (code_transitions, built only from the oracle's nearest rule)."""
    N = int(np.float32(1.0).view(np.uint32)) + 1           # bit patterns 0 .. 1.0
    per = 2047
    nblk = -(-N // per)
    say(f"exhaustive sweep kind={kind}: {N} values in {nblk} blocks")
    x = torch.zeros(nblk * 2048, dtype=torch.float32, device="cuda")
    xv = x.view(nblk, 2048)
    xv[:, 0] = 1.0
    sweep = torch.zeros(nblk * per, dtype=torch.float32, device="cuda")
    sweep[:N] = torch.arange(0, N, dtype=torch.int32, device="cuda").view(torch.float32)
    xv[:, 1:] = sweep.view(nblk, per)
    del sweep
    T = oracle.code_transitions(kind)
    want_pos = T.view(np.uint32).astype(np.int64)          # sweep index == bit pattern
    nmag = T.size + 1
    for sign in ([1.0, -1.0] if kind == oracle.SIGNED else [1.0]):
        if sign < 0:
            xv[:, 1:].neg_()
        codes, absmax = q.qopt_quantize_blockwise(x, kind)
        assert bool((absmax == 1.0).all())
        sc = codes.view(nblk, 2048)[:, 1:].reshape(-1)[:N]
        mag = (sc & 0x7F) if kind == oracle.SIGNED else sc
        change = torch.nonzero(mag[1:] != mag[:-1]).flatten() + 1
        got_pos = change.cpu().numpy()
        assert np.array_equal(got_pos, want_pos), (got_pos[:5], want_pos[:5])
        steps = (mag[change].int() - mag[change - 1].int()).cpu().numpy()
        assert np.all(steps == 1)
        assert int(mag[0]) == 0 and int(mag[-1]) == nmag - 1
        if kind == oracle.SIGNED:
            signs = (sc & 0x80) != 0
            if sign > 0:
                assert not bool(signs.any())
            else:   # every negative value carries the sign bit; -0.0 does not
                assert not bool(signs[0]) and bool(signs[1:].all())
        torch.cuda.synchronize()
    del x, codes, absmax
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", KINDS)
def test_full_size_student_t(q, kind):
    """2^28 values 0.01 * Student-t(3) (|x| for the unsigned codebook): sampled
    blocks against the oracle, and every block's absmax against torch.amax."""
    n = 1 << 28
    nblk = n // 2048
    say(f"full-size codec kind={kind} n={n}")
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    workloads.student_t3_(x, seed=1)
    if kind == oracle.UNSIGNED:
        x.abs_()
    codes, absmax = q.qopt_quantize_blockwise(x, kind)
    y = q.qopt_dequantize_blockwise(codes, absmax, kind)
    amax = x.view(nblk, 2048).abs().amax(dim=1)
    assert torch.equal(absmax, amax)
    sample = workloads.sample_blocks(nblk, 1500, seed=kind)
    idx = torch.from_numpy(sample).cuda()
    xs = x.view(nblk, 2048)[idx].cpu().numpy().reshape(-1)
    cs = codes.view(nblk, 2048)[idx].cpu().numpy().reshape(-1)
    ys = y.view(nblk, 2048)[idx].cpu().numpy().reshape(-1)
    c_ref, a_ref = oracle.quantize_blockwise(xs, kind)
    assert np.array_equal(cs, c_ref)
    assert np.array_equal(absmax[idx].cpu().numpy(), a_ref)
    assert np.array_equal(ys.view(np.uint32),
                          oracle.dequantize_blockwise(c_ref, a_ref, kind).view(np.uint32))
    del x, codes, absmax, y, amax
    torch.cuda.empty_cache()


def test_codec_past_32_bit_element_offsets(q):
    """One tensor of 2^32 + 3 * 2048 + 77 values (signed codebook), so that element
    offsets pass 2^31 and 2^32 and the last block is short: blocks on either side of
    both boundaries, the tail block and a random sample against the oracle."""
    kind = oracle.SIGNED
    n = (1 << 32) + 3 * 2048 + 77
    nblk = -(-n // 2048)
    say(f"codec past 32-bit offsets n={n}")
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    workloads.student_t3_(x, seed=9)
    codes, absmax = q.qopt_quantize_blockwise(x, kind)
    y = q.qopt_dequantize_blockwise(codes, absmax, kind)
    b31, b32 = (1 << 31) // 2048, (1 << 32) // 2048
    must = [0, b31 - 1, b31, b32 - 1, b32, nblk - 2, nblk - 1]
    for b in workloads.sample_blocks(nblk, 200, seed=3, must=must):
        b = int(b)
        lo, hi = b * 2048, min(n, b * 2048 + 2048)
        xs = x[lo:hi].cpu().numpy()
        c_ref, a_ref = oracle.quantize_blockwise(xs, kind)
        assert np.array_equal(codes[lo:hi].cpu().numpy(), c_ref), f"block {b}"
        assert absmax[b].item() == a_ref[0], f"block {b}"
        assert np.array_equal(y[lo:hi].cpu().numpy().view(np.uint32),
                              oracle.dequantize_blockwise(c_ref, a_ref, kind).view(np.uint32)), \
            f"block {b}"
    del x, codes, absmax, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", KINDS)
def test_multi_tensor_codec_matches_oracle(q, kind):
    """Many tensors (ragged tails, empty ones, misaligned views, more than 48 of them)
    in one multi-tensor call each way: every tensor equals the oracle's codec."""
    rng = np.random.default_rng(31 + kind)
    sizes = [int(s) for s in rng.integers(0, 9000, 70)] + [0, 1, 2048, 2049, 50257]
    xs = [workloads.student_t3_host(n, seed=1000 + i) for i, n in enumerate(sizes)]
    if kind == oracle.UNSIGNED:
        xs = [np.abs(x) for x in xs]
    buf = torch.zeros(sum(sizes) + 2 * len(sizes), dtype=torch.float32, device="cuda")
    cbuf = torch.zeros(sum(sizes) + 3 * len(sizes), dtype=torch.uint8, device="cuda")
    triples, off, coff = [], 0, 0
    for i, (n, x) in enumerate(zip(sizes, xs)):
        off += i % 2            # odd tensors start one element later: no vector path
        coff += i % 3
        v = buf[off:off + n]
        v.copy_(torch.from_numpy(x).cuda())
        triples.append((v, cbuf[coff:coff + n],
                        torch.full((-(-n // 2048),), -1.0, device="cuda")))
        off += n
        coff += n
    say(f"multi codec kind={kind}: {len(sizes)} tensors")
    q.qopt_quantize_blockwise_multi(triples, kind)
    ys = [torch.full_like(v, -7.0) for v, _, _ in triples]
    q.qopt_dequantize_blockwise_multi([(y, c, a) for y, (_, c, a) in zip(ys, triples)], kind)
    torch.cuda.synchronize()
    for i, (x, (v, c, a), y) in enumerate(zip(xs, triples, ys)):
        c_ref, a_ref = oracle.quantize_blockwise(x, kind)
        assert np.array_equal(c.cpu().numpy(), c_ref), i
        assert np.array_equal(a.cpu().numpy().view(np.uint32), a_ref.view(np.uint32)), i
        y_ref = oracle.dequantize_blockwise(c_ref, a_ref, kind)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32)), i
