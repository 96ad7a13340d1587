"""CPU parity of the C++ allocator's swapping (host pool, swap-out/in) with
the oracle allocator: the same block pairs, errors and pool states after
every operation."""
import numpy as np
import pytest

import oracle.allocator as OAL

P = pytest.importorskip("paged_kv_cache_292_amd", reason="libpkv.so not built")

_ERR = {OAL.OutOfBlocks: "OUT_OF_BLOCKS", OAL.NotFound: "NOT_FOUND",
        OAL.SharedWrite: "SHARED_WRITE", OAL.InvalidArg: "INVALID_ARG",
        OAL.Swapped: "SWAPPED"}


def _pair(n, nh, bs, fo=None, hfo=None):
    o, p = OAL.BlockAllocator(n, bs, fo), P.Allocator(n, bs, fo)
    o.set_host_pool(nh, hfo)
    p.set_host_pool(nh, hfo)
    return o, p


def _run(o, p, name_o, name_p, *args):
    """One operation on both sides: same result or the same error."""
    res_o = res_p = err_o = err_p = None
    try:
        res_o = getattr(o, name_o)(*args)
    except OAL.AllocatorError as e:
        err_o = _ERR[type(e)]
    try:
        res_p = getattr(p, name_p)(*args)
    except P.PkvError as e:
        err_p = e.code
    assert err_o == err_p, (name_o, args, err_o, err_p)
    return res_o, res_p, err_o


def _same_state(o, p, ids):
    assert o.num_free_blocks() == p.num_free_blocks()
    assert len(o.host_free) == p.num_free_host_blocks()
    for b in range(o.num_blocks):
        assert o.block_refcount(b) == p.block_refcount(b)
    for b in range(o.num_host_blocks):
        assert o.host_refcount[b] == p.host_block_refcount(b)
    for s in ids:
        if s not in o.tables:
            assert p.is_swapped(s) == -1
            continue
        assert p.is_swapped(s) == (1 if s in o.swapped else 0)
        assert p.num_blocks_of(s) == len(o.tables[s]) and p.context_len(s) == o.lengths[s]
    live = [s for s in ids if s in o.tables and s not in o.swapped]
    if live:
        mb = max(len(o.tables[s]) for s in live) + 1
        to, co = o.build_block_tables(live, mb)
        tp, cp = p.build_block_tables(live, mb)
        assert np.array_equal(to, tp) and np.array_equal(co, cp)


def test_hand_traced_example_in_cpp():
    o, p = _pair(8, 5, 4, [3, 7, 1, 0, 5, 2, 6, 4], [4, 2, 0, 3, 1])
    for a in (o, p):
        a.add(0); a.append(0, 10)
        a.add(1); a.fork_prefix(0, 1, 8)
        a.append(1, 2)
        a.add(2); a.fork_prefix(0, 2, 4)
    assert [tuple(r) for r in p.swap_out([1, 0])] == o.swap_out([1, 0]) == \
        [(3, 4), (7, 2), (0, 0), (1, 3)]
    _same_state(o, p, range(3))
    assert [tuple(r) for r in p.swap_in([0])] == o.swap_in([0]) == [(4, 5), (2, 2), (3, 6)]
    assert [tuple(r) for r in p.swap_in([1])] == o.swap_in([1]) == [(4, 4), (2, 0), (0, 7)]
    _same_state(o, p, range(3))


def test_errors_match_and_change_nothing():
    o, p = OAL.BlockAllocator(6, 4), P.Allocator(6, 4)
    for a in (o, p):
        a.add(0); a.append(0, 5)
        a.add(1); a.append(1, 9)
    _run(o, p, "swap_out", "swap_out", [0])            # no host pool: INVALID_ARG
    o.set_host_pool(2); p.set_host_pool(2)
    with pytest.raises(P.PkvError) as e:
        p.set_host_pool(2)
    assert e.value.code == "INVALID_ARG"
    for args in ([0, 1], [1], [0, 0], [0, 9], []):
        _run(o, p, "swap_out", "swap_out", args)
    _same_state(o, p, range(3))
    _run(o, p, "swap_in", "swap_in", [0])              # not swapped: SWAPPED
    _run(o, p, "swap_out", "swap_out", [0])
    _same_state(o, p, range(3))
    _run(o, p, "append", "append", 0, 1)
    with pytest.raises(P.PkvError) as e:
        p.append_cow([0], [1])
    assert e.value.code == "SWAPPED"
    _run(o, p, "add", "add", 2)
    _run(o, p, "fork_prefix", "fork_prefix", 0, 2, 4)
    _run(o, p, "fork_prefix", "fork_prefix", 1, 0, 0)
    with pytest.raises(P.PkvError) as e:
        p.build_block_tables([0], 4)
    assert e.value.code == "SWAPPED"
    seqs = np.array([0], dtype=np.int64)
    with pytest.raises(P.PkvError) as e:
        p.decode_step_prepare(seqs, 8, np.empty(1, np.int64), np.empty((1, 8), np.int32),
                              np.empty(1, np.int32))
    assert e.value.code == "SWAPPED"
    _run(o, p, "append", "append", 2, 4 * (o.num_free_blocks() - 1))
    _run(o, p, "swap_in", "swap_in", [0])              # one device block short
    _same_state(o, p, range(3))
    _run(o, p, "free_seq", "free", 0)                  # releases host blocks
    _same_state(o, p, range(3))


@pytest.mark.parametrize("seed", range(30))
def test_random_walk_matches_oracle(seed):
    rng = np.random.default_rng(2000 + seed)
    bs = int(rng.choice([1, 4, 16]))
    n, nh = int(rng.integers(8, 40)), int(rng.integers(4, 40))
    o, p = _pair(n, nh, bs, rng.permutation(n), rng.permutation(nh))
    next_id = 0
    moved = 0
    for _ in range(80):
        resident = [s for s in o.tables if s not in o.swapped]
        swapped = sorted(o.swapped)
        r = rng.random()
        if r < 0.15 or not resident:
            _run(o, p, "add", "add", next_id)
            next_id += 1
        elif r < 0.40:
            x, k = int(rng.choice(resident)), int(rng.integers(1, 2 * bs + 2))
            ro, rp, err = _run(o, p, "append", "append", x, k)
            if err is None:
                assert list(ro) == list(rp)
        elif r < 0.48:
            x, k = int(rng.choice(resident)), int(rng.integers(1, 2 * bs + 2))
            try:
                ro = o.append_cow(x, k)
                err_o = None
            except OAL.AllocatorError as e:
                err_o = _ERR[type(e)]
            try:
                rp = p.append_cow([x], [k])
                err_p = None
            except P.PkvError as e:
                err_p = e.code
            assert err_o == err_p
            if err_o is None:
                assert list(ro[0]) == list(rp[0]) and ro[1] == [tuple(t) for t in rp[1]]
        elif r < 0.56:
            src = int(rng.choice(resident))
            L = o.lengths[src]
            k = L if rng.random() < 0.5 else (L // bs) * bs
            _run(o, p, "add", "add", next_id)
            _run(o, p, "fork_prefix", "fork_prefix", src, next_id, k)
            next_id += 1
        elif r < 0.76:
            # mostly distinct resident ids; sometimes an id twice, an unknown id
            # or a swapped one: the errors must match too
            if rng.random() < 0.7:
                g = [int(x) for x in rng.choice(resident, size=min(len(resident), int(rng.integers(1, 4))),
                                                replace=False)]
            else:
                g = [int(x) for x in rng.choice(list(o.tables) + [999], size=int(rng.integers(1, 4)))]
            ro, rp, err = _run(o, p, "swap_out", "swap_out", g)
            if err is None:
                assert ro == [tuple(t) for t in rp]
                moved += len(ro)
        elif r < 0.93:
            pool = swapped if swapped and rng.random() < 0.9 else list(o.tables)
            if not pool:
                continue
            g = [int(x) for x in rng.choice(pool, size=min(len(pool), int(rng.integers(1, 4))),
                                            replace=False)]
            ro, rp, err = _run(o, p, "swap_in", "swap_in", g)
            if err is None:
                assert ro == [tuple(t) for t in rp]
                moved += len(ro)
        else:
            _run(o, p, "free_seq", "free", int(rng.choice(list(o.tables))))
        _same_state(o, p, range(next_id + 1))
    assert moved > 0


def test_swap_blocks_rejects_bad_arguments_before_any_gpu_call():
    """Argument checks that return before the HIP runtime is touched."""
    lib = P.lib
    fake = 0x10000
    assert lib.pkv_swap_blocks(fake, fake, fake, fake, fake, 1, 4, 4, 16, 2, 64, 1, 7, None) == -1
    assert lib.pkv_swap_blocks(fake, fake, fake, fake, fake, 1, 4, 4, 16, 2, 64, 5, 0, None) == -1
    assert lib.pkv_swap_blocks(fake, fake, fake, fake, fake, -1, 4, 4, 16, 2, 64, 1, 0, None) == -1
    assert lib.pkv_swap_blocks(fake, fake, fake, fake, fake, 0, 4, 4, 16, 2, 64, 1, 0, None) == 0
    assert lib.pkv_swap_blocks(fake, fake, None, fake, fake, 1, 4, 4, 16, 2, 64, 1, 1, None) == -1
    assert lib.pkv_swap_blocks(fake, fake, fake + 8, fake, fake, 1, 4, 4, 16, 2, 64, 1, 1, None) == -1
    assert lib.pkv_swap_blocks(fake, fake, fake, fake, fake, 1, 4, 4, 1, 1, 2, 1, 1, None) == -2
