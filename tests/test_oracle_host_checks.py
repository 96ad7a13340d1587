"""Pins of the oracle's shared-prefix member list (test infrastructure).

Sequences with a common prefix point at the same physical blocks ("What Is
vLLM …", section "How does PagedAttention work?", memory-sharing step).  The
oracle allocator's ``shared_prefix_members`` reports the largest group of
sequences, longer than the prefix, whose first prefix blocks are the same
physical blocks.  Pinned here by what fixes it independently: the workload
that builds the sharing by construction, a hand-traced fork tree, and
brute force over every group on random fork walks."""
import itertools

import numpy as np
import pytest

import oracle.allocator as OAL
import workloads as W


def members(a, seqs, prefix):
    return a.shared_prefix_members(list(seqs), prefix)


def test_gqa_batch_members_are_the_sharers_it_forked():
    """The GQA decode batch forks 128 of 256 sequences from one 1,024-token
    prefix; every other sequence owns all its blocks."""
    s = W.shape(3)
    wl = W.make_workload(s, with_payload=False)
    a = OAL.BlockAllocator(wl.num_blocks, s.block_size, wl.free_order)
    a.replay(wl.ops)
    assert members(a, range(s.num_seqs), s.shared_prefix_tokens) == list(wl.sharers)


def test_hand_traced_fork_tree():
    """Block size 4.  Sequence 0 holds 12 tokens (blocks A B C); 1 and 2 fork
    its first 8 (A B) and grow; 3 forks its first 4 (A) and grows; 4 owns
    its blocks; 5 forks A B and stops at 8 tokens (not longer than an
    8-token prefix)."""
    a = OAL.BlockAllocator(64, 4)
    for i in range(6):
        a.add(i)
    a.append(0, 12)
    a.fork_prefix(0, 1, 8)
    a.append(1, 3)
    a.fork_prefix(0, 2, 8)
    a.append(2, 9)
    a.fork_prefix(0, 3, 4)
    a.append(3, 6)
    a.append(4, 20)
    a.fork_prefix(0, 5, 8)
    batch = [0, 1, 2, 3, 4, 5]
    assert members(a, batch, 4) == [0, 1, 2, 3, 5]      # A
    assert members(a, batch, 8) == [0, 1, 2]            # A B, and 5 is not longer than 8
    assert members(a, batch, 12) == []                  # C is sequence 0's alone
    assert members(a, [4, 3, 2], 4) == [1, 2]           # positions in the batch given
    assert members(a, [4, 5], 8) == []                  # one sequence is no group
    # two groups of two: the one met first in the batch
    b = OAL.BlockAllocator(64, 4)
    for i in range(4):
        b.add(i)
    b.append(0, 5)
    b.append(1, 5)
    b.fork_prefix(0, 2, 4)
    b.append(2, 1)
    b.fork_prefix(1, 3, 4)
    b.append(3, 1)
    assert members(b, [0, 1, 2, 3], 4) == [0, 2]
    assert members(b, [3, 1, 2, 0], 4) == [0, 1]
    with pytest.raises(OAL.InvalidArg):
        members(b, [0, 1], 6)  # not a multiple of the block size
    with pytest.raises(OAL.InvalidArg):
        members(b, [0, 0], 4)


@pytest.mark.parametrize("seed", range(20))
def test_members_against_brute_force_over_every_group(seed):
    """On random fork walks: every member is longer than the prefix and
    holds the same first prefix blocks as the others; no group of sequences
    sharing their first prefix blocks is larger; among groups as large, none
    starts earlier in the batch."""
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([2, 4]))
    B = int(rng.integers(2, 10))
    a = OAL.BlockAllocator(400, bs)
    for i in range(B):
        a.add(i)
    nsrc = int(rng.integers(1, 3))
    for src in range(nsrc):
        a.append(src, int(rng.integers(1, 5)) * bs)
    for b in range(nsrc, B):
        if rng.random() < 0.7:
            src = int(rng.integers(0, nsrc))
            a.fork_prefix(src, b, int(rng.integers(1, a.lengths[src] // bs + 1)) * bs)
        a.append(b, int(rng.integers(0, 3 * bs)))
    batch = [int(x) for x in rng.permutation(B)]
    for nb in range(1, 5):
        pre = nb * bs
        got = members(a, batch, pre)
        key = {i: tuple(a.tables[s][:nb]) for i, s in enumerate(batch) if a.lengths[s] > pre}
        sizes = {}
        for i, k in key.items():
            sizes.setdefault(k, []).append(i)
        best = max((len(v) for v in sizes.values()), default=0)
        if best < 2:
            assert got == []
            continue
        assert len(got) == best and got == sorted(got)
        assert len({key[i] for i in got}) == 1
        first = min(min(v) for v in sizes.values() if len(v) == best)
        assert got[0] == first
        for i, j in itertools.combinations(got, 2):
            assert a.tables[batch[i]][:nb] == a.tables[batch[j]][:nb]


PINS = [
    test_gqa_batch_members_are_the_sharers_it_forked,
    test_hand_traced_fork_tree,
] + [lambda s=s: test_members_against_brute_force_over_every_group(s) for s in range(6)]
