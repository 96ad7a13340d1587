"""Pins of the allocator oracle: the pages' worked numbers and the invariants
their description fixes."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle.allocator as OAL
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_worked_example_960_vs_16384():
    g = _load("kv_slots_worked_example.json")
    bs = g["block_size"]
    outs = g["output_tokens"]
    a = OAL.BlockAllocator(num_blocks=1000, block_size=bs)
    for i, n in enumerate(outs):
        a.add(i)
        slots = a.append(i, g["prompt_tokens"] + n)
        assert len(set(slots)) == len(slots)
    used_blocks = a.num_blocks - a.num_free_blocks()
    assert used_blocks * bs == g["printed_paged_slots"] == 960
    assert [len(a.table(i)) for i in range(len(outs))] == [7, 9, 7, 7, 9, 7, 7, 7]
    assert len(outs) * g["max_context"] == g["printed_naive_slots"] == 16384
    # waste sits only in each sequence's last block
    for i, n in enumerate(outs):
        assert 0 <= len(a.table(i)) * bs - (g["prompt_tokens"] + n) < bs


def test_block_lookup_example():
    g = _load("block_lookup_example.json")
    e = g["blocks_for_100_tokens"]
    a = OAL.BlockAllocator(64, e["block_size"])
    a.add(0)
    a.append(0, 100)
    assert len(a.table(0)) == e["blocks"] == OAL.blocks_for(100, e["block_size"])
    for p in g["position_47"]:
        bs = p["block_size"]
        al = OAL.BlockAllocator(16, bs, free_order=W.permutation(3, 16))
        al.add(7)
        slots = al.append(7, 48)
        t = al.table(7)
        assert (47 // bs, 47 % bs) == (p["logical_block"], p["offset"])
        assert slots[47] == t[p["logical_block"]] * bs + p["offset"]
        assert slots[47] // bs == t[p["logical_block"]] and slots[47] % bs == p["offset"]


def test_fifo_policy_and_free_order():
    a = OAL.BlockAllocator(6, 4, free_order=[5, 2, 0, 4, 1, 3])
    a.add(1)
    a.add(2)
    assert a.append(1, 5) == [20, 21, 22, 23, 8]
    assert a.append(2, 1) == [0]
    a.free_seq(1)  # releases 5 then 2, appended to the tail
    assert list(a.free) == [4, 1, 3, 5, 2]
    assert a.append(2, 4) == [1, 2, 3, 16]


def test_errors_leave_state_unchanged():
    a = OAL.BlockAllocator(4, 16)
    a.add(0)
    a.append(0, 40)  # 3 blocks
    a.add(1)
    a.fork_prefix(0, 1, 32)
    snap = (list(a.free), list(a.refcount), {k: list(v) for k, v in a.tables.items()}, dict(a.lengths))
    with pytest.raises(OAL.OutOfBlocks):
        a.append(0, 100)
    with pytest.raises(OAL.NotFound):
        a.append(9, 1)
    with pytest.raises(OAL.InvalidArg):
        a.add(0)
    with pytest.raises(OAL.InvalidArg):
        a.fork_prefix(0, 1, 16)  # dst not empty
    a.add(2)
    with pytest.raises(OAL.InvalidArg):
        a.fork_prefix(0, 2, 8)  # neither whole blocks nor all of the source
    a.free_seq(2)
    # exhaustion exactly one block past what is free
    e = OAL.BlockAllocator(3, 4)
    e.add(0); e.append(0, 2)
    with pytest.raises(OAL.OutOfBlocks):
        e.append(0, 2 + 8 + 1)
    assert e.num_free_blocks() == 2 and e.context_len(0) == 2
    assert len(e.append(0, 2 + 8)) == 10 and e.num_free_blocks() == 0
    b = OAL.BlockAllocator(4, 16)
    b.add(0); b.append(0, 8); b.add(1)
    b.fork_prefix(0, 1, 0)
    assert (list(a.free), list(a.refcount), {k: list(v) for k, v in a.tables.items()}, dict(a.lengths)) == snap


def test_shared_write_refused():
    a = OAL.BlockAllocator(8, 4)
    a.add(0); a.append(0, 6)
    a.add(1); a.fork_prefix(0, 1, 4)
    # seq 1 ends on a block boundary: its next token opens a private block
    assert a.append(1, 1) == [a.table(1)[1] * 4]
    # seq 0's last block is private, writing into it is fine
    a.append(0, 1)
    # a full fork shares seq 0's partly filled last block: neither may write into it
    a.add(2); a.fork_prefix(0, 2, 7)
    assert a.block_refcount(a.table(0)[1]) == 2
    snap = (list(a.free), list(a.refcount))
    with pytest.raises(OAL.SharedWrite):
        a.append(0, 1)
    with pytest.raises(OAL.SharedWrite):
        a.append(2, 3)
    assert (list(a.free), list(a.refcount)) == snap
    a.append(2, 0)  # zero tokens: nothing is written
    a.free_seq(0)
    a.append(2, 1)  # the block is private again
    c = OAL.BlockAllocator(8, 4)
    c.add(0); c.append(0, 8)
    c.add(1); c.fork_prefix(0, 1, 8)
    c.free_seq(0)
    c.add(2); c.fork_prefix(1, 2, 8)
    assert c.block_refcount(c.table(1)[1]) == 2
    # a sequence whose last block is shared and full opens a new block: allowed
    assert len(c.append(2, 1)) == 1


def test_build_block_tables():
    a = OAL.BlockAllocator(10, 4, free_order=list(range(9, -1, -1)))
    for s, n in [(3, 5), (1, 0), (7, 9)]:
        a.add(s); a.append(s, n)
    t, c = a.build_block_tables([7, 1, 3], max_blocks=4, pad=-1)
    assert c.tolist() == [9, 0, 5]
    assert t.tolist() == [[7, 6, 5, -1], [-1] * 4, [9, 8, -1, -1]]
    with pytest.raises(OAL.InvalidArg):
        a.build_block_tables([7], max_blocks=2)


OPS = st.lists(st.tuples(st.sampled_from(["add", "append", "fork", "free"]),
                         st.integers(0, 5), st.integers(0, 5), st.integers(0, 40)),
               max_size=60)


@settings(max_examples=200, deadline=None)
@given(ops=OPS, bs=st.sampled_from([1, 4, 16]), n=st.integers(0, 24))
def test_invariants_random_ops(ops, bs, n):
    a = OAL.BlockAllocator(n, bs, free_order=W.permutation(n + 7, n) if n else None)
    for op, x, y, k in ops:
        try:
            if op == "add":
                a.add(x)
            elif op == "append":
                before = a.context_len(x) if x in a.lengths else None
                slots = a.append(x, k)
                t = a.table(x)
                for i, s in enumerate(slots):
                    pos = before + i
                    assert s == t[pos // bs] * bs + pos % bs
            elif op == "fork":
                a.fork_prefix(x, y, k)
            else:
                a.free_seq(x)
        except OAL.AllocatorError:
            pass
        live = {}
        for s, t in a.tables.items():
            assert len(t) == OAL.blocks_for(a.lengths[s], bs)  # waste only in the last block
            for blk in t:
                live[blk] = live.get(blk, 0) + 1
        assert len(a.free) + len(live) == n  # conservation
        assert set(a.free).isdisjoint(live)
        for blk in range(n):
            assert a.refcount[blk] == live.get(blk, 0)
    for s in list(a.tables):
        a.free_seq(s)
    assert sorted(a.free) == list(range(n))


def test_workload_replay_shapes():
    """Replaying each decode shape's op list gives each sequence its context and
    the prefix blocks the expected reference counts."""
    for i in range(5):
        s = W.shape(i)
        if i in (3, 4):
            s = W.scaled(s, num_seqs=24 if i == 3 else 3, num_sharers=8 if i == 3 else None)
        wl = W.make_workload(s, with_payload=False)
        a = OAL.BlockAllocator(wl.num_blocks, s.block_size, wl.free_order)
        a.replay(wl.ops)
        if s.new_tokens:
            for b in range(s.num_seqs):
                a.append(b, 1)
        for b in range(s.num_seqs):
            assert a.context_len(b) == wl.ctx[b]
        assert a.num_free_blocks() == (64 - 13 if i == 0 else 0)
        if s.num_sharers:
            pre = a.table(int(wl.sharers[0]))[: s.shared_prefix_tokens // s.block_size]
            for blk in pre:
                assert a.block_refcount(blk) == s.num_sharers
            for b in wl.sharers:
                assert a.table(int(b))[: len(pre)] == pre
