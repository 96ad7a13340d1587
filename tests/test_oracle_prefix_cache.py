"""Pins of the prefix-cache oracle (requests with the same prefix share its
physical blocks: "Serving models with vLLM", section "How it works:
PagedAttention"; "What Is vLLM …", memory-sharing step).

What any correct prefix cache must satisfy, checked against models that know
nothing of the cache: a shared block holds exactly the keys and values the new
request would have computed for those positions (a synthetic model whose rows
depend only on token and position stands in for the network); with no
eviction, a prompt shares as many full blocks as the longest prefix it has in
common with an earlier prompt (brute force over all earlier prompts); both
counts and the free list stay consistent.  Block ids follow the first-in
first-out reading, pinned by a hand-traced example."""
import numpy as np
import pytest

import oracle.allocator as OAL
import oracle.attention as OA
import oracle.cache_write as OC


def test_hand_traced_example():
    a = OAL.BlockAllocator(12, 4)
    a.enable_prefix_cache()
    A = list(range(1, 11))                       # 10 tokens: blocks 0, 1 full, 2 partial
    assert a.add_prompt(0, A) == (list(range(10)), 0)
    B = list(range(1, 9)) + [20, 21]             # shares blocks 0 and 1
    assert a.add_prompt(1, B) == ([12, 13], 8)
    assert a.table(1) == [0, 1, 3]
    C = [1, 2, 3, 4, 9, 9, 9, 9]                 # 8 tokens: only block 0 may be shared
    assert a.add_prompt(2, C) == ([16, 17, 18, 19], 4)
    assert a.prefix_cache_stats() == (5, 3, 3)
    a.free_seq(0)                                # 2 -> free
    a.free_seq(1)                                # 1, 3 -> free (1 keeps its entry)
    assert list(a.free) == [5, 6, 7, 8, 9, 10, 11, 2, 1, 3]
    D = list(range(1, 9)) + [30]                 # revives block 1 from the free list
    assert a.add_prompt(3, D) == ([20], 8)
    assert a.table(3) == [0, 1, 5] and a.block_refcount(1) == 1
    assert list(a.free) == [6, 7, 8, 9, 10, 11, 2, 3]
    a.free_seq(2)                                # 4 -> free, entry kept
    a.free_seq(3)                                # 0, 1, 5 -> free, entries kept
    assert list(a.free) == [6, 7, 8, 9, 10, 11, 2, 3, 4, 0, 1, 5]
    assert a.prefix_cache_stats() == (7, 5, 3)
    F = list(range(100, 136))                    # 9 fresh blocks: pops ... 3, 4 (4 evicted)
    slots, cached = a.add_prompt(5, F)
    assert cached == 0 and a.table(5) == [6, 7, 8, 9, 10, 11, 2, 3, 4]
    assert a.prefix_cache_stats() == (15, 5, 2 + 9)
    G = [200, 201, 202, 203]                     # pops 0: drops (1..4) and its child (1..8)
    assert a.add_prompt(6, G) == ([0, 1, 2, 3], 0)
    assert a.prefix_cache_stats() == (15, 5, 9 + 1)
    H = list(range(1, 9))                        # block 1 still holds 1..8 but is unreachable
    assert a.add_prompt(7, H) == ([4, 5, 6, 7, 20, 21, 22, 23], 0)
    assert a.table(7) == [1, 5]
    assert a.prefix_cache_stats() == (16, 5, 12)


def test_last_token_is_never_shared():
    """A prompt that is a whole number of blocks, all cached, still computes
    its last block; the cached copy keeps the entry."""
    a = OAL.BlockAllocator(8, 4)
    a.enable_prefix_cache()
    P = [1, 2, 3, 4, 5, 6, 7, 8]
    assert a.add_prompt(0, P) == (list(range(8)), 0)
    assert a.add_prompt(1, P) == ([8, 9, 10, 11], 4)    # block 1 computed again, in block 2
    assert a.table(1) == [0, 2]
    assert a.add_prompt(2, P + [9]) == ([12], 8)        # finds the first copy, block 1
    assert a.table(2) == [0, 1, 3]
    assert a.prefix_cache_stats() == (4, 3, 2)
    assert a.add_prompt(3, [5]) == ([16], 0)            # a one-token prompt: nothing to look up
    assert a.prefix_cache_stats() == (4, 3, 2)


def test_disabled_cache_and_errors():
    a = OAL.BlockAllocator(6, 4)
    assert a.add_prompt(0, [5] * 9) == (list(range(9)), 0)
    assert a.add_prompt(1, [5] * 9) == (list(range(12, 21)), 0)   # no sharing when disabled
    assert a.prefix_cache_stats() == (0, 0, 0)
    with pytest.raises(OAL.InvalidArg):
        a.add_prompt(1, [1])
    a.enable_prefix_cache()
    with pytest.raises(OAL.InvalidArg):
        a.enable_prefix_cache()
    a.free_seq(0)
    a.free_seq(1)
    a.add_prompt(2, [7] * 8)                     # 2 blocks, both entered
    a.free_seq(2)                                # both free, entries kept
    snap = lambda: (list(a.free), list(a.refcount), dict(a.prefix_cache), a.prefix_cache_stats(),
                    {k: list(v) for k, v in a.tables.items()})
    before = snap()
    # shares block 0 (revived from the free list), then needs 6 more: 5 left
    with pytest.raises(OAL.OutOfBlocks):
        a.add_prompt(3, [7] * 4 + [1] * 21)
    assert snap() == before
    assert a.add_prompt(3, [7] * 4 + [1] * 20)[1] == 4
    assert a.num_free_blocks() == 0


def _rows(tokens, positions, H, D):
    """Synthetic model: the K and V rows of a token depend only on its id and
    its position (fixed per-id and per-position patterns)."""
    tok = np.asarray(tokens, dtype=np.float64)[:, None, None]
    pos = np.asarray(positions, dtype=np.float64)[:, None, None]
    h = np.arange(H)[None, :, None]
    d = np.arange(D)[None, None, :]
    k = np.sin(0.37 * tok + 0.011 * pos * (d + 1) + h)
    v = np.cos(0.53 * tok - 0.007 * pos * (d + 2) + 2 * h)
    return k, v


def _check_cache_contents(a, kc, vc, H, D):
    bs = a.block_size
    for key, blk in a.prefix_cache.items():
        j = len(key) // bs - 1
        k, v = _rows(key[j * bs:], range(j * bs, (j + 1) * bs), H, D)
        assert np.array_equal(kc[blk], k) and np.array_equal(vc[blk], v), key
        assert a.block_key[blk] == key


@pytest.mark.parametrize("seed", range(25))
def test_shared_blocks_hold_the_right_rows(seed):
    """Prompts built from a few shared prefixes (system prompts, documents)
    plus unique tails, with frees, decode appends and forks between them: after
    every operation each sequence's rows, read through its table, are the
    synthetic model's rows of its own tokens, and every cached block holds the
    rows of the prefix it is cached under."""
    rng = np.random.default_rng(300 + seed)
    bs = int(rng.choice([2, 4, 8]))
    H, D = 1, 3
    N = int(rng.integers(12, 40))
    a = OAL.BlockAllocator(N, bs, free_order=rng.permutation(N))
    a.enable_prefix_cache()
    kc = np.full((N, bs, H, D), np.nan)
    vc = np.full((N, bs, H, D), np.nan)
    prefixes = [list(rng.integers(0, 50, size=int(rng.integers(1, 4 * bs)))) for _ in range(4)]
    toks = {}
    next_id = 0
    for _ in range(50):
        r = rng.random()
        live = list(a.tables)
        if r < 0.5 or not live:
            base = prefixes[int(rng.integers(0, len(prefixes)))]
            cut = int(rng.integers(0, len(base) + 1))
            prompt = base[:cut] + list(rng.integers(0, 50, size=int(rng.integers(0, 2 * bs + 1))))
            if not prompt:
                continue
            try:
                slots, cached = a.add_prompt(next_id, prompt)
            except OAL.OutOfBlocks:
                continue
            k, v = _rows(prompt[cached:], range(cached, len(prompt)), H, D)
            kc, vc = OC.reshape_and_cache(k, v, kc, vc, slots)
            toks[next_id] = list(prompt)
            next_id += 1
        elif r < 0.7:
            s = int(rng.choice(live))
            n = int(rng.integers(1, bs + 2))
            new = list(rng.integers(0, 50, size=n))
            try:
                slots = a.append(s, n)
            except OAL.AllocatorError:
                continue
            k, v = _rows(new, range(len(toks[s]), len(toks[s]) + n), H, D)
            kc, vc = OC.reshape_and_cache(k, v, kc, vc, slots)
            toks[s] += new
        elif r < 0.8:
            s = int(rng.choice(live))
            L = a.context_len(s)
            k_tok = (L // bs) * bs
            a.add(next_id)
            a.fork_prefix(s, next_id, k_tok)
            toks[next_id] = toks[s][:k_tok]
            next_id += 1
        else:
            s = int(rng.choice(live))
            a.free_seq(s)
            del toks[s]
        for s, t in toks.items():
            gk = OA.gather_sequence(kc, a.tables[s], a.lengths[s], bs)
            gv = OA.gather_sequence(vc, a.tables[s], a.lengths[s], bs)
            k, v = _rows(t, range(len(t)), H, D)
            assert len(t) == a.lengths[s]
            if t:
                assert np.array_equal(gk, k) and np.array_equal(gv, v)
        _check_cache_contents(a, kc, vc, H, D)
        live_blocks = {}
        for t in a.tables.values():
            for b in t:
                live_blocks[b] = live_blocks.get(b, 0) + 1
        assert len(a.free) + len(live_blocks) == N and set(a.free).isdisjoint(live_blocks)
        assert all(a.refcount[b] == live_blocks.get(b, 0) for b in range(N))


@pytest.mark.parametrize("seed", range(10))
def test_sharing_is_maximal_without_eviction(seed):
    """With a pool large enough that nothing is evicted, each prompt shares
    exactly the full blocks of its longest common prefix with any earlier
    prompt (never its last token): brute force over all earlier prompts."""
    rng = np.random.default_rng(700 + seed)
    bs = int(rng.choice([1, 2, 4]))
    a = OAL.BlockAllocator(4000, bs)
    a.enable_prefix_cache()
    seen = []
    bases = [list(rng.integers(0, 3, size=12)) for _ in range(3)]
    for i in range(40):
        b = bases[int(rng.integers(0, 3))]
        p = b[: int(rng.integers(0, 13))] + list(rng.integers(0, 3, size=int(rng.integers(0, 6))))
        if not p:
            continue
        best = 0
        for q in seen:
            m = 0
            while m < min(len(p), len(q)) and p[m] == q[m]:
                m += 1
            # q's blocks up to its own length were entered (full blocks only)
            best = max(best, min(m, (len(q) // bs) * bs))
        expect = min((best // bs) * bs, ((len(p) - 1) // bs) * bs)
        _, cached = a.add_prompt(i, p)
        assert cached == expect, (p, cached, expect)
        seen.append(p)


def test_prefill_with_shared_system_prompt_equals_unshared():
    """Chunked prefill of requests that share a system prompt: attending over
    the shared blocks gives exactly the output of the same requests laid out
    without sharing."""
    rng = np.random.default_rng(9)
    bs, H, D = 4, 2, 8
    system = list(rng.integers(0, 100, size=22))
    prompts = [system + list(rng.integers(0, 100, size=int(n))) for n in (3, 7, 1, 12)]
    outs = []
    for share in (True, False):
        a = OAL.BlockAllocator(64, bs, free_order=rng.permutation(64))
        if share:
            a.enable_prefix_cache()
        kc = np.zeros((64, bs, H, D))
        vc = np.zeros((64, bs, H, D))
        starts, qrows = [0], []
        for i, p in enumerate(prompts):
            slots, cached = a.add_prompt(i, p)
            assert cached == (20 if share and i else 0)
            k, v = _rows(p[cached:], range(cached, len(p)), H, D)
            kc, vc = OC.reshape_and_cache(k, v, kc, vc, slots)
            # the queries are the last 3 tokens of each prompt
            qk, _ = _rows(p[-3:], range(len(p) - 3, len(p)), 2 * H, D)
            qrows.append(qk)
            starts.append(starts[-1] + 3)
        tables, ctx = a.build_block_tables(list(range(len(prompts))), 16)
        if share:
            assert len(set(tables[:, 0])) == 1  # the system prompt's first block is shared
        outs.append(OA.paged_prefill(np.concatenate(qrows).astype(np.float32), kc, vc, tables, ctx,
                                     np.array(starts), 0.3, "f32"))
    np.testing.assert_array_equal(outs[0], outs[1])


# cheapest first: a planted mistake is reported by the first pin that fails
PINS = [test_hand_traced_example, test_last_token_is_never_shared, test_disabled_cache_and_errors,
        test_prefill_with_shared_system_prompt_equals_unshared]
PINS += [lambda s=s: test_sharing_is_maximal_without_eviction(s) for s in range(0, 10, 3)]
PINS += [lambda s=s: test_shared_blocks_hold_the_right_rows(s) for s in range(0, 25, 3)]
