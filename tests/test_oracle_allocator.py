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


OPS = st.lists(st.tuples(st.sampled_from(["add", "append", "fork", "free", "cow"]),
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
            elif op == "cow":
                held = a.table(x)[-1] if x in a.tables and a.tables[x] else None
                shared = held is not None and a.refcount[held] > 1
                slots, pairs = a.append_cow(x, k)
                for src, dst in pairs:
                    assert src == held and shared and a.refcount[dst] == 1
                t = a.table(x)
                for pos, s_ in zip(range(a.context_len(x) - k, a.context_len(x)), slots):
                    assert s_ == t[pos // bs] * bs + pos % bs
                    assert a.refcount[t[pos // bs]] == 1  # never written while shared
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


def test_copy_on_write_append():
    """Beam candidates fork a whole sequence and then diverge: the first writer
    into the shared, partly filled last block gets a private copy; the last
    holder writes in place; full shared blocks are never copied."""
    a = OAL.BlockAllocator(10, 4, free_order=list(range(10)))
    a.add(0); a.append(0, 6)                  # blocks [0, 1], 2 tokens in block 1
    a.add(1); a.fork_prefix(0, 1, 6)          # full fork: shares 0 and 1
    assert a.block_refcount(1) == 2
    slots, pairs = a.append_cow(0, 3)         # seq 0 copies block 1 -> 2, appends 3 tokens
    assert pairs == [(1, 2)]
    assert a.table(0) == [0, 2, 3] and a.table(1) == [0, 1]
    assert slots == [2 * 4 + 2, 2 * 4 + 3, 3 * 4 + 0]
    assert a.block_refcount(1) == 1 and a.block_refcount(2) == 1 and a.block_refcount(0) == 2
    slots, pairs = a.append_cow(1, 1)         # seq 1 now holds block 1 alone: no copy
    assert pairs == [] and slots == [1 * 4 + 2]
    # a shared block that is full is not copied: the next token opens a new block
    a.add(2); a.fork_prefix(1, 2, 4)
    slots, pairs = a.append_cow(2, 1)
    assert pairs == [] and a.table(2) == [0, 4] and slots == [16]
    # zero tokens: nothing copied
    a.add(3); a.fork_prefix(0, 3, 9)
    assert a.append_cow(3, 0) == ([], [])
    # pool exhaustion counts the copy, and leaves everything unchanged
    free = a.num_free_blocks()
    snap = (list(a.free), list(a.refcount), {k: list(v) for k, v in a.tables.items()})
    with pytest.raises(OAL.OutOfBlocks):
        a.append_cow(3, 3 + 4 * free)
    assert (list(a.free), list(a.refcount), {k: list(v) for k, v in a.tables.items()}) == snap
    assert len(a.append_cow(3, 3 + 4 * (free - 1))[1]) == 1
