"""Pins of the swap oracle (preemption by swapping a sequence's KV blocks to a
host pool and back: "What Is vLLM …", section "What is continuous batching in
vLLM?", step 2).

The pages fix only that a preempted sequence's cache leaves the GPU for CPU
memory and comes back; the pins check what that implies for any correct
implementation (every token's K/V row is the same before and after, both
pools conserve their blocks, reference counts equal the number of holders),
against a logical model that keeps each sequence's rows in a plain list and
knows nothing of blocks.  The block ids come from the first-in first-out
reading of the free lists, pinned by a hand-traced example."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle.allocator as OAL
import oracle.attention as OA
import oracle.cache_write as OC


def test_hand_traced_example():
    """Sharing inside and outside the swapped group, traced by hand from the
    reading: visiting order = sequence by sequence in table order; one host
    block per distinct device block; freed blocks go to the free list's tail."""
    a = OAL.BlockAllocator(8, 4, free_order=[3, 7, 1, 0, 5, 2, 6, 4])
    a.set_host_pool(5, host_free_order=[4, 2, 0, 3, 1])
    a.add(0); a.append(0, 10)          # A = [3, 7, 1]
    a.add(1); a.fork_prefix(0, 1, 8)   # B shares [3, 7]
    a.append(1, 2)                     # B = [3, 7, 0]
    a.add(2); a.fork_prefix(0, 2, 4)   # C = [3]
    assert [a.refcount[b] for b in (3, 7, 1, 0)] == [3, 2, 1, 1]
    # B first: 3 -> h4, 7 -> h2, 0 -> h0 (0 is freed); then A: 3 and 7 reuse
    # h4 and h2 (7 is freed, 3 stays with C), 1 -> h3 (freed)
    assert a.swap_out([1, 0]) == [(3, 4), (7, 2), (0, 0), (1, 3)]
    assert a.table(1) == [4, 2, 0] and a.table(0) == [4, 2, 3] and a.table(2) == [3]
    assert list(a.free) == [5, 2, 6, 4, 0, 7, 1]
    assert list(a.host_free) == [1]
    assert [a.host_refcount[h] for h in range(5)] == [1, 0, 2, 1, 2]
    assert a.refcount[3] == 1
    # A back alone: h4 -> 5, h2 -> 2, h3 -> 6 (h3 freed; h4, h2 still held by B)
    assert a.swap_in([0]) == [(4, 5), (2, 2), (3, 6)]
    assert a.table(0) == [5, 2, 6] and list(a.host_free) == [1, 3]
    # then B: h4 -> 4, h2 -> 0, h0 -> 7, all host blocks freed in that order
    assert a.swap_in([1]) == [(4, 4), (2, 0), (0, 7)]
    assert a.table(1) == [4, 0, 7] and list(a.free) == [1]
    assert list(a.host_free) == [1, 3, 4, 2, 0]
    assert a.lengths == {0: 10, 1: 10, 2: 4} and not a.swapped


def test_swapped_sequences_are_frozen_and_errors_change_nothing():
    a = OAL.BlockAllocator(6, 4)
    with pytest.raises(OAL.InvalidArg):      # no host pool yet
        a.swap_out([])
    a.set_host_pool(2)
    with pytest.raises(OAL.InvalidArg):
        a.set_host_pool(2)
    a.add(0); a.append(0, 5)                 # 2 blocks
    a.add(1); a.append(1, 9)                 # 3 blocks
    snap = lambda: (list(a.free), list(a.refcount), list(a.host_free), list(a.host_refcount),
                    {k: list(v) for k, v in a.tables.items()}, set(a.swapped))
    before = snap()
    with pytest.raises(OAL.OutOfBlocks):     # 5 distinct blocks, 2 host blocks
        a.swap_out([0, 1])
    with pytest.raises(OAL.OutOfBlocks):     # 3 blocks: one short
        a.swap_out([1])
    with pytest.raises(OAL.InvalidArg):
        a.swap_out([0, 0])
    with pytest.raises(OAL.NotFound):
        a.swap_out([0, 9])
    with pytest.raises(OAL.Swapped):
        a.swap_in([0])
    assert snap() == before
    assert a.swap_out([0]) == [(0, 0), (1, 1)]
    for call in (lambda: a.append(0, 1), lambda: a.append_cow(0, 1),
                 lambda: a.fork_prefix(0, 1, 4), lambda: a.build_block_tables([0], 4),
                 lambda: a.swap_out([0])):
        with pytest.raises(OAL.Swapped):
            call()
    a.add(2)
    with pytest.raises(OAL.Swapped):         # fork into or out of a swapped sequence
        a.fork_prefix(0, 2, 4)
    # the device pool is one block short for a swap-in: nothing changes
    a.append(2, 4 * (len(a.free) - 1))
    assert len(a.free) == 1
    before = snap()
    with pytest.raises(OAL.OutOfBlocks):
        a.swap_in([0])
    assert snap() == before
    a.free_seq(0)                            # releases its host blocks
    assert sorted(a.host_free) == [0, 1] and a.host_refcount == [0, 0]


def _check_pools(a: OAL.BlockAllocator, n: int, nh: int) -> None:
    """Conservation and reference counts on both pools."""
    live, hlive = {}, {}
    for s, t in a.tables.items():
        assert len(t) == OAL.blocks_for(a.lengths[s], a.block_size)
        tgt = hlive if s in a.swapped else live
        for b in t:
            tgt[b] = tgt.get(b, 0) + 1
    assert len(a.free) + len(live) == n and set(a.free).isdisjoint(live)
    assert len(a.host_free) + len(hlive) == nh and set(a.host_free).isdisjoint(hlive)
    assert all(a.refcount[b] == live.get(b, 0) for b in range(n))
    assert all(a.host_refcount[b] == hlive.get(b, 0) for b in range(nh))


class _World:
    """The paged model (oracle allocator, device cache, host pool, block
    moves) next to a logical model that keeps each sequence's rows as a plain
    list."""

    def __init__(self, n, nh, bs, rng):
        self.rng, self.n, self.nh, self.bs = rng, n, nh, bs
        self.H, self.D = 1, 2
        self.a = OAL.BlockAllocator(n, bs, free_order=rng.permutation(n))
        self.a.set_host_pool(nh, host_free_order=rng.permutation(nh))
        shape = (bs, self.H, self.D)
        self.kd, self.vd = rng.standard_normal((n,) + shape), rng.standard_normal((n,) + shape)
        self.kh, self.vh = rng.standard_normal((nh,) + shape), rng.standard_normal((nh,) + shape)
        self.logical = {}  # seq -> list of (k row, v row)

    def apply(self, op, x=0, y=0, k=0, group=()):
        a, rng = self.a, self.rng
        try:
            if op == "add":
                a.add(x)
                self.logical[x] = []
            elif op in ("append", "cow"):
                if op == "append":
                    slots, pairs = a.append(x, k), []
                else:
                    slots, pairs = a.append_cow(x, k)
                for s_, d_ in pairs:
                    self.kd[d_], self.vd[d_] = self.kd[s_], self.vd[s_]
                new_k = rng.standard_normal((k, self.H, self.D))
                new_v = rng.standard_normal((k, self.H, self.D))
                self.kd, self.vd = OC.reshape_and_cache(new_k, new_v, self.kd, self.vd, slots)
                self.logical[x] += list(zip(new_k, new_v))
            elif op == "fork":
                a.fork_prefix(x, y, k)
                self.logical[y] = list(self.logical[x][:k])
            elif op == "free":
                a.free_seq(x)
                del self.logical[x]
            elif op == "out":
                pairs = a.swap_out(list(group))
                self.kh, self.vh = OC.move_blocks(self.kd, self.vd, self.kh, self.vh, pairs)
                for b in a.free:  # freed device blocks may be handed out again
                    self.kd[b] = np.nan
                    self.vd[b] = np.nan
                return pairs
            else:
                pairs = a.swap_in(list(group))
                self.kd, self.vd = OC.move_blocks(self.kh, self.vh, self.kd, self.vd, pairs)
                for b in a.host_free:
                    self.kh[b] = np.nan
                    self.vh[b] = np.nan
                return pairs
        except OAL.AllocatorError:
            return None
        return []

    def check(self):
        a = self.a
        _check_pools(a, self.n, self.nh)
        for s, rows in self.logical.items():
            kc, vc = (self.kh, self.vh) if s in a.swapped else (self.kd, self.vd)
            gk = OA.gather_sequence(kc, a.tables[s], a.lengths[s], self.bs)
            gv = OA.gather_sequence(vc, a.tables[s], a.lengths[s], self.bs)
            assert len(rows) == a.lengths[s]
            for t, (rk, rv) in enumerate(rows):
                assert np.array_equal(gk[t], rk) and np.array_equal(gv[t], rv)


OPS = st.lists(st.tuples(st.sampled_from(["append", "append", "fork", "free", "cow", "out", "out",
                                          "in", "in", "add"]),
                         st.integers(0, 4), st.integers(0, 4), st.integers(0, 9),
                         st.lists(st.integers(0, 4), min_size=1, max_size=3)),
               max_size=40)


@settings(max_examples=200, deadline=None)
@given(ops=OPS, bs=st.sampled_from([1, 2, 4]), n=st.integers(4, 24), nh=st.integers(2, 16),
       seed=st.integers(0, 2**16))
def test_rows_survive_swapping(ops, bs, n, nh, seed):
    """Random workloads with swaps: after every operation, every sequence's
    rows read through its table, from the device cache if resident or the
    host pool if swapped, equal its logical rows; both pools conserve blocks."""
    w = _World(n, nh, bs, np.random.default_rng(seed))
    for s in range(5):
        w.apply("add", s)
    for op, x, y, k, group in ops:
        w.apply(op, x, y, k, list(dict.fromkeys(group)))
        w.check()


@pytest.mark.parametrize("seed", range(40))
def test_rows_survive_swapping_random_walk(seed):
    """The same check on seeded walks that pick valid targets (resident
    sequences to grow, fork or swap out; swapped ones to swap in), so most
    swaps move blocks, shared ones included."""
    rng = np.random.default_rng(1000 + seed)
    bs = int(rng.choice([1, 2, 4]))
    w = _World(32, 24, bs, rng)
    moved = 0
    next_id = 0
    for _ in range(60):
        a = w.a
        resident = [s for s in a.tables if s not in a.swapped]
        swapped = sorted(a.swapped)
        r = rng.random()
        if r < 0.15 or not resident:
            w.apply("add", next_id)
            next_id += 1
        elif r < 0.45:
            w.apply(rng.choice(["append", "cow"]), int(rng.choice(resident)),
                    k=int(rng.integers(1, 3 * bs + 1)))
        elif r < 0.55:
            src = int(rng.choice(resident))
            L = a.lengths[src]
            k = L if rng.random() < 0.5 else (L // bs) * bs
            w.apply("add", next_id)
            w.apply("fork", src, next_id, k)
            next_id += 1
        elif r < 0.75:
            g = rng.choice(resident, size=min(len(resident), int(rng.integers(1, 4))), replace=False)
            pairs = w.apply("out", group=[int(x) for x in g])
            moved += len(pairs or [])
        elif r < 0.92 and swapped:
            g = rng.choice(swapped, size=min(len(swapped), int(rng.integers(1, 4))), replace=False)
            pairs = w.apply("in", group=[int(x) for x in g])
            moved += len(pairs or [])
        else:
            w.apply("free", int(rng.choice(list(a.tables))))
        w.check()
    assert moved > 0


def test_decode_unchanged_by_a_swap_round_trip():
    """A swapped-out and swapped-in batch decodes to exactly the same output,
    with the freed device blocks reused and overwritten in between."""
    rng = np.random.default_rng(5)
    N, bs, H, D, NH = 24, 4, 2, 8, 20
    a = OAL.BlockAllocator(N, bs, free_order=rng.permutation(N))
    a.set_host_pool(NH)
    kd = rng.standard_normal((N, bs, H, D))
    vd = rng.standard_normal((N, bs, H, D))
    kh = np.zeros((NH, bs, H, D))
    vh = np.zeros((NH, bs, H, D))
    for s, L in enumerate([9, 13, 5]):
        a.add(s)
        a.append(s, L)
    a.add(3); a.fork_prefix(1, 3, 8); a.append(3, 3)
    q = rng.standard_normal((4, 2 * H, D))
    seqs = [0, 1, 2, 3]
    t0, c0 = a.build_block_tables(seqs, 6)
    ref = OA.paged_decode(q, kd, vd, t0, c0, 0.3, "f32")
    pairs = a.swap_out([1, 3])
    assert len(pairs) == len({*a.tables[1], *a.tables[3]})  # the shared prefix is copied once
    kh, vh = OC.move_blocks(kd, vd, kh, vh, pairs)
    a.add(9)
    slots = a.append(9, bs * len(a.free))  # another sequence takes every free block
    kd, vd = OC.reshape_and_cache(rng.standard_normal((len(slots), H, D)),
                                  rng.standard_normal((len(slots), H, D)), kd, vd, slots)
    a.free_seq(9)
    kd, vd = OC.move_blocks(kh, vh, kd, vd, a.swap_in([3, 1]))
    t1, c1 = a.build_block_tables(seqs, 6)
    assert not np.array_equal(t0, t1)
    assert np.array_equal(OA.paged_decode(q, kd, vd, t1, c1, 0.3, "f32"), ref)


# cheapest first: a planted mistake is reported by the first pin that fails
PINS = [test_hand_traced_example, test_swapped_sequences_are_frozen_and_errors_change_nothing,
        test_decode_unchanged_by_a_swap_round_trip]
PINS += [lambda s=s: test_rows_survive_swapping_random_walk(s) for s in range(0, 40, 4)]
PINS += [test_rows_survive_swapping]
