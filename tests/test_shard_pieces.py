"""The per-rank share used to time the step at one rank's shape (CPU only).

Blocks are independent, so a rank that owns a contiguous range of whole 2048-blocks
of the flattened tensors steps its share with no communication. These checks pin the
split that ``workloads.shard_pieces`` computes:
- the ranks' pieces tile every tensor exactly, in order;
- every piece starts on a block boundary of its tensor;
- block counts differ by at most one between ranks.
"""

import numpy as np
import pytest

import workloads
from workloads import BLOCK, nblocks, shard_pieces


def _check_split(sizes, world):
    total = sum(nblocks(n) for n in sizes)
    flat = []                                 # (tensor, first, count) over all ranks in order
    counts = []
    for r in range(world):
        pieces = shard_pieces(sizes, world, r)
        counts.append(sum(nblocks(c) for _, _, c in pieces))
        for i, e0, c in pieces:
            assert c > 0 and e0 % BLOCK == 0 and e0 + c <= sizes[i]
        flat += pieces
    assert sum(counts) == total
    assert max(counts) - min(counts) <= 1
    assert counts == sorted(counts, reverse=True)   # the longer ranges come first
    # in rank order the pieces walk every tensor from its first to its last element
    expect_i, expect_e = 0, 0
    for i, e0, c in flat:
        while expect_i < len(sizes) and expect_e == sizes[expect_i]:
            expect_i, expect_e = expect_i + 1, 0
        assert (i, e0) == (expect_i, expect_e)
        expect_e = e0 + c
    while expect_i < len(sizes) and expect_e == sizes[expect_i]:
        expect_i, expect_e = expect_i + 1, 0
    assert expect_i == len(sizes)


@pytest.mark.parametrize("world", [1, 2, 3, 7, 8, 9])
def test_random_tensor_lists(world):
    rng = np.random.default_rng(world)
    for _ in range(20):
        k = int(rng.integers(1, 40))
        sizes = [int(s) for s in (10 ** rng.uniform(0, 5, k)).astype(np.int64)]
        for j in rng.choice(k, size=k // 5, replace=False):
            sizes[j] = 0                      # empty tensors own no blocks
        _check_split(sizes, world)


def test_more_ranks_than_blocks():
    sizes = [1, 2048, 2049]                   # 4 blocks
    _check_split(sizes, 6)
    assert shard_pieces(sizes, 6, 5) == [] and shard_pieces(sizes, 6, 4) == []
    assert shard_pieces(sizes, 6, 0) == [(0, 0, 1)]
    assert shard_pieces(sizes, 6, 3) == [(2, 2048, 1)]


def test_llama7b_eighth():
    sizes = [n for _, n in workloads.llama7b_shapes()]
    _check_split(sizes, 8)
    p0 = shard_pieces(sizes, 8, 0)
    assert sum(nblocks(c) for _, _, c in p0) == 411_281     # ceil(3,290,242 / 8)
    assert sum(c for _, _, c in p0) == 842_303_488 and len(p0) == 35
    assert p0[0] == (0, 0, 32000 * 4096)                      # the embedding, whole


def test_bad_rank():
    with pytest.raises(ValueError):
        shard_pieces([10], 2, 2)
