"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and lays out parameter shapes; it holds
none of the optimizer's or the codec's arithmetic, so both the HIP path and the
CPU oracle can consume what it produces.

Workloads (all synthetic; the pages' quality benchmarks need datasets and are
not throughput workloads):

* ``flat1m``     one fp32 tensor of 1,048,576 params; p ~ N(0, 0.02); fp32 grads
                 ~ N(0, 1e-3) drawn fresh per step with 0.1 % of the entries (1,049,
                 uniform without replacement) scaled by 100; 10 steps.
* ``codec256m``  2^28 fp32 values 0.01 * Student-t(3); the same values' absolute
                 values feed the unsigned codebook.
* ``gpt1p3b``    GPT-shaped 1.3B parameter set (24 layers, d 2048, ffn 8192, tied
                 50,257-token embedding, LayerNorm weight and bias vectors), 243
                 tensors; fp32 p ~ N(0, 0.02), bf16 g ~ N(0, 1e-3).
* ``llama7b``    Llama-shaped 7B parameter set (32 layers, d 4096, ffn 11008, 32,000
                 token embedding and untied head, RMSNorm vectors), 291 tensors;
                 fp32 p ~ N(0, 0.02), bf16 g ~ N(0, 1e-3) with 0.01 % of the entries
                 scaled by 1000.
* ``flat20b``    one flat bf16 buffer of 2e10 params updated in place; p ~ N(0, 0.02),
                 g ~ N(0, 5e-4); the first 256,000 x 4096 elements form an embedding
                 whose gradient rows are nonzero in 2 % of the rows (5,120 rows drawn
                 per step), zero elsewhere in that region.
* ``llama7b_shard8``  one rank's share of ``llama7b`` when 8 ranks split the 2048-blocks
                 of the flattened parameter set into contiguous ranges (rank 0: the
                 first 411,281 blocks, 842,303,488 params in 35 tensor pieces); same
                 value recipe and seed as ``llama7b``.
* ``embed7b``    the Stable Embedding layer at the Llama-7B embedding's shape: a
                 32,000 x 4096 table, 65,536 tokens (32 sequences of 2048) whose ids
                 follow Zipf's law with exponent 1 over the vocabulary (ranks mapped
                 to ids by a seeded permutation), bf16 outputs and bf16 upstream
                 gradients ~ N(0, 1).
"""

import numpy as np

BLOCK = 2048


# --------------------------------------------------------------------------- shapes

def gpt1p3b_shapes():
    """(name, numel) of the GPT-shaped 1.3B parameter set, 243 tensors."""
    d, ffn, vocab, layers = 2048, 8192, 50257, 24
    out = [("embed", vocab * d)]
    for i in range(layers):
        out += [(f"h{i}.ln1.w", d), (f"h{i}.ln1.b", d),
                (f"h{i}.q", d * d), (f"h{i}.k", d * d), (f"h{i}.v", d * d),
                (f"h{i}.o", d * d),
                (f"h{i}.ln2.w", d), (f"h{i}.ln2.b", d),
                (f"h{i}.fc1", ffn * d), (f"h{i}.fc2", d * ffn)]
    out += [("lnf.w", d), ("lnf.b", d)]
    return out


def llama7b_shapes():
    """(name, numel) of the Llama-shaped 7B parameter set, 291 tensors."""
    d, ffn, vocab, layers = 4096, 11008, 32000, 32
    out = [("embed", vocab * d)]
    for i in range(layers):
        out += [(f"l{i}.attn_norm", d),
                (f"l{i}.q", d * d), (f"l{i}.k", d * d), (f"l{i}.v", d * d),
                (f"l{i}.o", d * d),
                (f"l{i}.ffn_norm", d),
                (f"l{i}.gate", ffn * d), (f"l{i}.up", ffn * d), (f"l{i}.down", d * ffn)]
    out += [("norm", d), ("lm_head", vocab * d)]
    return out


FLAT20B_N = 20_000_000_000
FLAT20B_EMBED_ROWS = 256_000
FLAT20B_EMBED_DIM = 4096
FLAT20B_ACTIVE_ROWS = 5_120  # 2 % of the rows

HPARAMS = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def nblocks(n):
    return -(-int(n) // BLOCK)


def shard_pieces(sizes, world, rank):
    """Rank ``rank``'s share when ``world`` ranks split the 2048-blocks of the
    flattened tensors (blocks counted per tensor, the last one of a tensor may be
    short) into contiguous ranges, the first ``total % world`` ranks one block
    longer: a list of (tensor index, first element, element count), every first
    element a multiple of 2048 within its tensor."""
    if not 0 <= rank < world:
        raise ValueError(f"rank {rank} outside 0..{world - 1}")
    nbs = [nblocks(n) for n in sizes]
    total = sum(nbs)
    per, extra = divmod(total, world)
    lo = rank * per + min(rank, extra)
    hi = lo + per + (1 if rank < extra else 0)
    out, first = [], 0                    # first: global index of the tensor's block 0
    for i, (n, nb) in enumerate(zip(sizes, nbs)):
        a, b = max(lo, first), min(hi, first + nb)
        if a < b:
            e0 = (a - first) * BLOCK
            out.append((i, e0, min(int(n), (b - first) * BLOCK) - e0))
        first += nb
    return out


# ---------------------------------------------------------------------- host (numpy)

def flat1m(n=1_048_576, steps=10, seed=0, outlier_frac=0.001, outlier_scale=100.0):
    """Host arrays for the flat fp32 workload: (p0, [g_step1, ..., g_stepK]).

    Drawn in this order from numpy's PCG64 seeded with ``seed``: p0, then per step
    the gradient and the outlier positions.
    """
    rng = np.random.default_rng(seed)
    p0 = rng.normal(0.0, 0.02, n).astype(np.float32)
    k = int(np.ceil(outlier_frac * n))
    grads = []
    for _ in range(steps):
        g = rng.normal(0.0, 1e-3, n).astype(np.float32)
        idx = rng.choice(n, size=k, replace=False)
        g[idx] *= np.float32(outlier_scale)
        grads.append(g)
    return p0, grads


def student_t3_host(n, seed=1, scale=0.01):
    """0.01 * Student-t(3) fp32 values on the host (numpy PCG64)."""
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_t(3, n)).astype(np.float32)


def host_normal(n, std, seed):
    return np.random.default_rng(seed).normal(0.0, std, n).astype(np.float32)


# ------------------------------------------------------------------- device (torch)

def _torch():
    import torch
    return torch


def device_generator(seed, device):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def fill_normal_(t, std, seed, chunk=1 << 27):
    """Fill a 1-D device tensor (fp32 or bf16) with N(0, std) from a seeded
    generator, in chunks so that no large fp32 temporary is needed."""
    torch = _torch()
    gen = device_generator(seed, t.device)
    n = t.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        tmp = torch.randn(e - s, generator=gen, device=t.device, dtype=torch.float32)
        tmp.mul_(std)
        t[s:e].copy_(tmp)
    return t


def scale_random_entries_(t, frac, factor, seed):
    """Multiply ``ceil(frac * n)`` entries of a 1-D device tensor, drawn uniformly
    (duplicates removed), by ``factor``."""
    torch = _torch()
    n = t.numel()
    k = int(np.ceil(frac * n))
    if k == 0:
        return t
    gen = device_generator(seed, t.device)
    idx = torch.randint(0, n, (k,), generator=gen, device=t.device, dtype=torch.int64)
    idx = torch.unique(idx)
    t[idx] = (t[idx].float() * factor).to(t.dtype)
    return t


def student_t3_(t, seed, scale=0.01, chunk=1 << 26):
    """Fill a 1-D fp32 device tensor with scale * Student-t(3), drawn as
    z / sqrt((z1^2 + z2^2 + z3^2) / 3) from independent standard normals."""
    torch = _torch()
    gen = device_generator(seed, t.device)
    n = t.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        z = torch.randn(4, e - s, generator=gen, device=t.device, dtype=torch.float32)
        chi2 = z[1].square() + z[2].square() + z[3].square()
        t[s:e] = scale * z[0] / torch.sqrt(chi2 / 3.0)
    return t


def sparse_rows_mask(rows, active, seed, device):
    """Boolean mask over ``rows`` rows with ``active`` rows set, chosen uniformly
    without replacement."""
    torch = _torch()
    gen = device_generator(seed, device)
    perm = torch.randperm(rows, generator=gen, device=device)[:active]
    mask = torch.zeros(rows, dtype=torch.bool, device=device)
    mask[perm] = True
    return mask


EMBED7B = dict(rows=32000, dim=4096, ntokens=65536)


def zipf_token_ids(ntokens, vocab, seed, exponent=1.0):
    """int64 token ids: rank k (1-based) has probability proportional to k^-exponent,
    and ranks are mapped to ids by a seeded permutation of the vocabulary."""
    rng = np.random.default_rng(seed)
    w = 1.0 / np.arange(1, vocab + 1, dtype=np.float64) ** exponent
    ranks = rng.choice(vocab, size=ntokens, p=w / w.sum())
    return rng.permutation(vocab).astype(np.int64)[ranks]


def sample_blocks(nblk, count, seed, must=()):
    """Sorted block indices for sampled parity: ``must`` plus ``count`` distinct blocks
    drawn uniformly without replacement (first and last blocks always included)."""
    rng = np.random.default_rng(seed)
    pick = set(int(b) for b in must if 0 <= int(b) < nblk)
    if nblk > 0:
        pick.update([0, nblk - 1])
    if nblk > 0 and count > 0:
        pick.update(int(b) for b in rng.choice(nblk, size=min(int(count), nblk), replace=False))
    return np.array(sorted(pick), dtype=np.int64)
