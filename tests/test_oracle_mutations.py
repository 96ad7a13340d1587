"""Planted mistakes in the oracle (on the CPU only) must each fail a pin.

Each case copies an oracle module's source, applies one plausible slip — a
swapped index, a dropped term, a flipped sign, a wrong operand — loads the
copy as a throwaway module and runs the pins against it."""
import os
import types

import pytest

import test_oracle_allocator as TAL
import test_oracle_attention as TA
import test_oracle_cache_write as TC
import test_oracle_host_checks as THC
import test_oracle_prefix_cache as TPC
import test_oracle_swap as TS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _mutant(rel, old, new):
    path = os.path.join(ROOT, rel)
    src = open(path).read()
    assert src.count(old) >= 1, (rel, old)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), path, "exec"), mod.__dict__)
    return mod


def _caught(pins, *args):
    for pin in pins:
        try:
            pin(*args)
        except (Exception, pytest.fail.Exception):
            return True
    return False


ATTN = [
    ("cache[int(table_row[t // block_size]), t % block_size]",
     "cache[int(table_row[t % block_size]), t // block_size]"),
    ("g = h // group", "g = h % group"),
    ("logits = scale * (k @ q)", "logits = (k @ q)"),
    ("return e / e.sum(axis=-1, keepdims=True)", "return e"),
    ("softmax_weights(logits) @ v", "softmax_weights(-logits) @ v"),
    ("softmax_weights(logits) @ v", "softmax_weights(logits) @ k"),
    ("<< 16", "<< 15"),
    ("for t in range(ctx)]", "for t in range(ctx - 1)]"),
    ("attend(qf[b, h], k[:, g, :], v[:, g, :], scale)", "attend(qf[b, h], k[:, g, :], v[:, 0, :], scale)"),
    ("attend(qf[b, h], k[:, g, :], v[:, g, :], scale)", "attend(qf[b, g], k[:, g, :], v[:, g, :], scale)"),
    ("z = logits - logits.max(axis=-1, keepdims=True)", "z = logits - logits.max(axis=-1, keepdims=True) * 0 + 1e-3 * logits"),
    ("return np.zeros(q_bh.shape[-1], dtype=np.float64)", "return np.ones(q_bh.shape[-1], dtype=np.float64)"),
    ("np.asarray(x, dtype=np.float32).astype(np.float64)", "np.asarray(x, dtype=np.float16).astype(np.float64)"),
    ("pos = ctx - n + i", "pos = ctx - n + i - 1"),
    ("k[: pos + 1, g, :], v[: pos + 1, g, :]", "k[:ctx, g, :], v[:ctx, g, :]"),
    ("out[lo + i, h] = attend(qf[lo + i, h]", "out[lo + i, h] = attend(qf[lo, h]"),
    ("            if pos < 0:\n                continue\n", "\n"),
]


@pytest.mark.parametrize("old,new", ATTN, ids=[f"attn{i}" for i in range(len(ATTN))])
def test_attention_mutant_caught(old, new):
    assert _caught(TA.PINS, _mutant("oracle/attention.py", old, new))


CW = [
    ("kc[slot // bs, slot % bs] = key[i]", "kc[slot % bs, slot // bs] = key[i]"),
    ("vc[slot // bs, slot % bs] = value[i]", "vc[slot // bs, slot % bs] = key[i]"),
    ("if slot < 0:\n            continue", "if slot < -1:\n            continue"),
    ("kc = k_cache.copy()", "kc = k_cache"),
]


@pytest.mark.parametrize("old,new", CW, ids=[f"cw{i}" for i in range(len(CW))])
def test_cache_write_mutant_caught(old, new):
    assert _caught(TC.PINS, _mutant("oracle/cache_write.py", old, new))


ALLOC = [
    ("return (num_tokens + block_size - 1) // block_size", "return num_tokens // block_size"),
    ("return int(table[pos // block_size]) * block_size + pos % block_size",
     "return int(table[pos // block_size]) * block_size + pos // block_size"),
    ("        blk = self.free.popleft()\n", "        blk = self.free.pop()\n"),
    ("self.free.append(blk)", "self.free.appendleft(blk)"),
    ("if pos % bs == 0:", "if pos % bs == 1:"),
    ("self.refcount[blk] -= 1", "self.refcount[blk] -= 2"),
    ("if n and length % bs and self.refcount[table[-1]] > 1:", "if n and length % bs and self.refcount[table[-1]] > 2:"),
    ("if need > len(self.free):", "if need > len(self.free) + 1:"),
    ("shared = self.tables[src][: blocks_for(num_tokens, bs)]", "shared = self.tables[src][: num_tokens // bs]"),
    ("tables[i, : len(t)] = t", "tables[i, : len(t)] = t[::-1]"),
    ("copy = n > 0 and length % bs != 0 and self.refcount[table[-1]] > 1",
     "copy = n > 0 and self.refcount[table[-1]] > 1"),
    ("            self.refcount[old] -= 1\n", "\n"),
    ("- len(table) + (1 if copy else 0)", "- len(table)"),
]

ALLOC_PINS = ["test_worked_example_960_vs_16384", "test_block_lookup_example",
              "test_fifo_policy_and_free_order", "test_errors_leave_state_unchanged",
              "test_shared_write_refused", "test_build_block_tables",
              "test_invariants_random_ops", "test_workload_replay_shapes",
              "test_copy_on_write_append"]


@pytest.mark.parametrize("old,new", ALLOC, ids=[f"alloc{i}" for i in range(len(ALLOC))])
def test_allocator_mutant_caught(old, new, monkeypatch):
    m = _mutant("oracle/allocator.py", old, new)
    monkeypatch.setattr(TAL, "OAL", m)
    assert _caught([getattr(TAL, n) for n in ALLOC_PINS])


SWAP_ALLOC = [
    ("                if blk not in to_host:\n", "                if True:\n"),
    ("to_host[blk] = self.host_free.popleft()", "to_host[blk] = self.host_free.pop()"),
    ("to_dev[blk] = self._take_free()", "to_dev[blk] = self.free.pop()"),
    ("                self.refcount[blk] -= 1\n                if self.refcount[blk] == 0:\n"
     "                    self.free.append(blk)\n                new_table.append(to_host[blk])",
     "                self.refcount[blk] -= 1\n                new_table.append(to_host[blk])"),
    ("                self.host_refcount[blk] -= 1\n                if self.host_refcount[blk] == 0:\n"
     "                    self.host_free.append(blk)\n                new_table.append(to_dev[blk])",
     "                new_table.append(to_dev[blk])"),
    ("            self.swapped.add(s)\n", "\n"),
    ("            self.swapped.discard(s)\n        return pairs", "\n        return pairs"),
    ("        self._resident(seq)\n        if n < 0:", "        if n < 0:"),
    ("if len(distinct) > len(self.host_free):", "if len(distinct) > len(self.host_free) + 1:"),
    ("        if seq in self.swapped:\n            self.swapped.discard(seq)",
     "        if False:\n            self.swapped.discard(seq)"),
    ("pairs.append((blk, to_host[blk]))", "pairs.append((to_host[blk], blk))"),
]


@pytest.mark.parametrize("old,new", SWAP_ALLOC, ids=[f"swapa{i}" for i in range(len(SWAP_ALLOC))])
def test_swap_allocator_mutant_caught(old, new, monkeypatch):
    monkeypatch.setattr(TS, "OAL", _mutant("oracle/allocator.py", old, new))
    assert _caught(TS.PINS)


SWAP_MOVE = [
    ("k[int(d)] = src_k[int(s)]", "k[int(s)] = src_k[int(d)]"),
    ("v[int(d)] = src_v[int(s)]", "v[int(d)] = src_k[int(s)]"),
    ("    k = dst_k.copy()\n", "    k = src_k.copy()\n"),
]


@pytest.mark.parametrize("old,new", SWAP_MOVE, ids=[f"swapm{i}" for i in range(len(SWAP_MOVE))])
def test_swap_move_mutant_caught(old, new, monkeypatch):
    monkeypatch.setattr(TS, "OC", _mutant("oracle/cache_write.py", old, new))
    assert _caught(TS.PINS)


PREFIX = [
    # the key is the block's own tokens, not the whole prefix
    ("blk = self.prefix_cache.get(tuple(tokens[: (j + 1) * bs]))",
     "blk = self.prefix_cache.get(tuple(tokens[j * bs: (j + 1) * bs]))"),
    ("                key = tuple(tokens[: (j + 1) * bs])\n",
     "                key = tuple(tokens[j * bs: (j + 1) * bs])\n"),
    # the last prompt token may be shared
    ("            for j in range(max(n - 1, 0) // bs):", "            for j in range(n // bs):"),
    # a revived block stays in the free list
    ("                self.free.remove(b)\n", "                pass\n"),
    # revived blocks are not counted against the free list
    ("need > len(self.free) - revived:", "need > len(self.free):"),
    # the entries extending an evicted block survive
    ("for k in [k for k in self.prefix_cache if k[: len(key)] == key]:",
     "for k in [k for k in self.prefix_cache if k == key]:"),
    # a handed-out block keeps its entry
    ("        if self.prefix_cache is not None and blk in self.block_key:\n",
     "        if False:\n"),
    # an existing entry is replaced by the new block
    ("                if key not in self.prefix_cache:\n", "                if True:\n"),
    # the partial last block is entered too
    ("            for j in range(len(hits), n // bs):", "            for j in range(len(hits), blocks_for(n, bs)):"),
    # hits are not counted
    ("            self.cache_hits += len(hits)\n", "\n"),
]


@pytest.mark.parametrize("old,new", PREFIX, ids=[f"prefix{i}" for i in range(len(PREFIX))])
def test_prefix_cache_mutant_caught(old, new, monkeypatch):
    monkeypatch.setattr(TPC, "OAL", _mutant("oracle/allocator.py", old, new))
    assert _caught(TPC.PINS)


MEMBERS = [
    # sequences no longer than the prefix counted as members
    ("            if self.lengths[s] > prefix_tokens:\n", "            if self.lengths[s] >= prefix_tokens:\n"),
    # grouped by one block too few
    ("groups.setdefault(tuple(self.tables[s][:nb]), []).append(i)",
     "groups.setdefault(tuple(self.tables[s][:nb - 1]), []).append(i)"),
    # a lone sequence reported as a group
    ("if len(g) >= 2 and len(g) > len(best):", "if len(g) >= 1 and len(g) > len(best):"),
    # the last group met wins a tie
    ("if len(g) >= 2 and len(g) > len(best):", "if len(g) >= 2 and len(g) >= len(best):"),
    # sequence ids instead of positions in the batch
    ("groups.setdefault(tuple(self.tables[s][:nb]), []).append(i)",
     "groups.setdefault(tuple(self.tables[s][:nb]), []).append(s)"),
]


@pytest.mark.parametrize("old,new", MEMBERS, ids=[f"members{i}" for i in range(len(MEMBERS))])
def test_shared_prefix_members_mutant_caught(old, new, monkeypatch):
    monkeypatch.setattr(THC, "OAL", _mutant("oracle/allocator.py", old, new))
    assert _caught(THC.PINS)
