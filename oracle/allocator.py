"""Oracle: the paged KV block allocator as a plain Python model.

What the pages fix:

* a sequence's cache is split into fixed-size blocks placed anywhere in the
  pool, and a per-sequence block table maps its logical blocks to physical
  ones, the way a page table maps pages ("vLLM in Production …", section
  "PagedAttention — Virtual Memory for the KV Cache"; "What Is vLLM …",
  section "How does PagedAttention work?", block allocation and block-table
  steps);
* blocks are taken one at a time as tokens arrive, so only the last block of a
  sequence is partly empty ("Serving models with vLLM", section
  "How it works: PagedAttention");
* sequences with a common prefix may point at the same physical blocks, kept
  alive by reference counting ("What Is vLLM …", memory-sharing step).

Readings where the pages are silent (also listed in the design notes):

* which free block comes next: a first-in first-out free list that starts as
  ``free_order`` (ascending ids when not given); freed blocks go to its tail in
  the order they are released (table order of the freed sequence);
* a fork shares the blocks holding the first ``num_tokens`` tokens of the
  source; ``num_tokens`` is a multiple of the block size, or the source's
  whole length (a full fork, as beam candidates do, which may share a
  partly filled last block);
* plain appending into a block that more than one sequence holds is refused;
  the copy-on-write append first gives the writer a private copy of that
  block (a fresh block from the free list, the shared block's count drops by
  one) and reports the (source, copy) pair so the caller copies the bytes
  ("What Is vLLM …", memory-sharing step: sharing by reference counts and
  copy-on-write);
* a failing call changes nothing.

Preemption by swapping ("What Is vLLM …", section "What is continuous
batching in vLLM?", step 2: under memory pressure low-priority sequences are
preempted and their KV caches moved to CPU memory).  The pages give no
mechanism; the reading here:

* a second pool of blocks in host memory, with its own first-in first-out
  free list (``host_free_order``, ascending ids when not given);
* ``swap_out(seqs)`` visits the sequences' device blocks sequence by
  sequence, in table order; each distinct block gets one host block (blocks
  shared inside the group stay shared), and the (device, host) pair is
  reported for the copy; each holder's reference moves to the host block, and
  a device block whose count drops to zero goes to the tail of the device
  free list (a block also held outside the group is copied but stays);
* ``swap_in(seqs)`` does the same in the other direction with fresh device
  blocks, reporting (host, device) pairs;
* a swapped-out sequence cannot grow, fork or be listed in block tables
  until it is swapped in; freeing it releases its host blocks.

Automatic prefix caching ("Serving models with vLLM", section "How it works:
PagedAttention": requests with the same prefix, such as a system prompt, point
at the same physical blocks, which is how prefix caching works; "What Is
vLLM …", memory-sharing step: sequences whose KV caches are identical share
blocks).  The pages give no mechanism; the reading here:

* a full block's keys and values are fixed by the tokens of the whole prefix
  that ends with it, so the cache maps that prefix (as a token tuple) to the
  block holding it;
* a new prompt shares the longest run of cached full blocks at its start,
  but never its last token (its keys and values are computed, so the prompt
  always has a query); a shared block that was free leaves the free list
  (order of the others kept) and is held again;
* the prompt's other full blocks are entered into the cache as they are
  allocated (the caller writes their keys and values before any later
  reader's attention runs); a key already present keeps its block;
* a freed block keeps its entry until the free list hands it out for other
  tokens; then its entry is dropped, and with it every entry whose prefix
  extends it (they could only be reached through it).

Token ``pos`` of a sequence is stored at slot ``table[pos // bs] * bs + pos % bs``.
Test infrastructure only.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = ["AllocatorError", "OutOfBlocks", "NotFound", "SharedWrite", "InvalidArg", "Swapped",
           "BlockAllocator", "slot_of", "blocks_for"]


class AllocatorError(Exception):
    pass


class OutOfBlocks(AllocatorError):
    pass


class NotFound(AllocatorError):
    pass


class SharedWrite(AllocatorError):
    pass


class InvalidArg(AllocatorError):
    pass


class Swapped(AllocatorError):
    """The sequence is swapped out (or, for a swap-in, is not)."""


def blocks_for(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` occupies: all full ones plus a partial one."""
    return (num_tokens + block_size - 1) // block_size


def slot_of(table: Sequence[int], pos: int, block_size: int) -> int:
    """Flat slot of token ``pos``: its physical block times the block size plus
    its row inside the block."""
    return int(table[pos // block_size]) * block_size + pos % block_size


class BlockAllocator:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Iterable[int]] = None):
        if num_blocks < 0 or block_size <= 0:
            raise InvalidArg("bad pool size or block size")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("free_order must be a permutation of the pool ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: deque = deque(order)
        self.refcount: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lengths: Dict[int, int] = {}
        # host pool for swapped-out sequences (absent until set)
        self.num_host_blocks: Optional[int] = None
        self.host_free: deque = deque()
        self.host_refcount: List[int] = []
        self.swapped: set = set()
        # prefix cache (absent until enabled): whole-prefix token tuple -> block
        self.prefix_cache: Optional[Dict[tuple, int]] = None
        self.block_key: Dict[int, tuple] = {}
        self.cache_lookups = 0
        self.cache_hits = 0

    def enable_prefix_cache(self) -> None:
        if self.prefix_cache is not None:
            raise InvalidArg("the prefix cache is already enabled")
        self.prefix_cache = {}

    def _take_free(self) -> int:
        """Hand out the block at the head of the free list.  A block that still
        held a cached prefix loses its entry, and so do the entries extending it."""
        blk = self.free.popleft()
        if self.prefix_cache is not None and blk in self.block_key:
            key = self.block_key[blk]
            for k in [k for k in self.prefix_cache if k[: len(key)] == key]:
                del self.block_key[self.prefix_cache.pop(k)]
        return blk

    def add_prompt(self, seq: int, tokens: Sequence[int]) -> Tuple[List[int], int]:
        """New sequence ``seq`` with prompt ``tokens``: shares the cached full
        blocks of its longest cached prefix (never the last token), allocates
        the rest, enters its other full blocks into the cache.  Returns the
        slots of the tokens after the shared part and the number of shared
        tokens."""
        if seq in self.tables:
            raise InvalidArg(f"sequence {seq} exists")
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        bs = self.block_size
        hits: List[int] = []
        if self.prefix_cache is not None:
            for j in range(max(n - 1, 0) // bs):
                blk = self.prefix_cache.get(tuple(tokens[: (j + 1) * bs]))
                if blk is None:
                    break
                hits.append(blk)
        revived = sum(1 for b in hits if self.refcount[b] == 0)
        need = blocks_for(n, bs) - len(hits)
        if need > len(self.free) - revived:
            raise OutOfBlocks(f"need {need} blocks, {len(self.free) - revived} free")
        for b in hits:
            if self.refcount[b] == 0:
                self.free.remove(b)
            self.refcount[b] += 1
        self.tables[seq] = list(hits)
        self.lengths[seq] = len(hits) * bs
        slots = self.append(seq, n - len(hits) * bs)
        if self.prefix_cache is not None:
            self.cache_lookups += max(n - 1, 0) // bs
            self.cache_hits += len(hits)
            for j in range(len(hits), n // bs):
                key = tuple(tokens[: (j + 1) * bs])
                if key not in self.prefix_cache:
                    self.prefix_cache[key] = self.tables[seq][j]
                    self.block_key[self.tables[seq][j]] = key
        return slots, len(hits) * bs

    def prefix_cache_stats(self) -> Tuple[int, int, int]:
        """(full-block lookups, hits, blocks holding a cached prefix)."""
        return self.cache_lookups, self.cache_hits, len(self.prefix_cache or {})

    def set_host_pool(self, num_host_blocks: int,
                      host_free_order: Optional[Iterable[int]] = None) -> None:
        if self.num_host_blocks is not None:
            raise InvalidArg("the host pool is already set")
        if num_host_blocks < 0:
            raise InvalidArg("negative host pool size")
        order = (list(range(num_host_blocks)) if host_free_order is None
                 else [int(b) for b in host_free_order])
        if sorted(order) != list(range(num_host_blocks)):
            raise InvalidArg("host_free_order must be a permutation of the host pool ids")
        self.num_host_blocks = num_host_blocks
        self.host_free = deque(order)
        self.host_refcount = [0] * num_host_blocks

    def _resident(self, seq: int) -> None:
        if seq not in self.tables:
            raise NotFound(seq)
        if seq in self.swapped:
            raise Swapped(f"sequence {seq} is swapped out")

    # -- queries -----------------------------------------------------------
    def num_free_blocks(self) -> int:
        return len(self.free)

    def block_refcount(self, block: int) -> int:
        if not 0 <= block < self.num_blocks:
            return -1
        return self.refcount[block]

    def table(self, seq: int) -> List[int]:
        if seq not in self.tables:
            raise NotFound(seq)
        return list(self.tables[seq])

    def context_len(self, seq: int) -> int:
        if seq not in self.lengths:
            raise NotFound(seq)
        return self.lengths[seq]

    # -- updates -----------------------------------------------------------
    def add(self, seq: int) -> None:
        if seq in self.tables:
            raise InvalidArg(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lengths[seq] = 0

    def append(self, seq: int, n: int) -> List[int]:
        """Grow ``seq`` by ``n`` tokens; returns their slots in order."""
        self._resident(seq)
        if n < 0:
            raise InvalidArg("negative token count")
        table = self.tables[seq]
        length = self.lengths[seq]
        bs = self.block_size
        need = blocks_for(length + n, bs) - len(table)
        if n and length % bs and self.refcount[table[-1]] > 1:
            raise SharedWrite(f"last block of sequence {seq} is shared")
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        slots = []
        for pos in range(length, length + n):
            if pos % bs == 0:
                blk = self._take_free()
                self.refcount[blk] += 1
                table.append(blk)
            slots.append(slot_of(table, pos, bs))
        self.lengths[seq] = length + n
        return slots

    def append_cow(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Grow ``seq`` by ``n`` tokens, copying a shared, partly filled last
        block first.  Returns (slots, copy pairs (source block, new block))."""
        self._resident(seq)
        if n < 0:
            raise InvalidArg("negative token count")
        table = self.tables[seq]
        length = self.lengths[seq]
        bs = self.block_size
        copy = n > 0 and length % bs != 0 and self.refcount[table[-1]] > 1
        need = blocks_for(length + n, bs) - len(table) + (1 if copy else 0)
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        pairs = []
        if copy:
            old = table[-1]
            new = self._take_free()
            self.refcount[new] += 1
            self.refcount[old] -= 1
            table[-1] = new
            pairs.append((old, new))
        return self.append(seq, n), pairs

    def fork_prefix(self, src: int, dst: int, num_tokens: int) -> None:
        """Make ``dst`` (empty) share the first ``num_tokens`` tokens of ``src``."""
        if src not in self.tables or dst not in self.tables:
            raise NotFound((src, dst))
        self._resident(src)
        self._resident(dst)
        bs = self.block_size
        whole = num_tokens % bs == 0 or num_tokens == self.lengths[src]
        if (num_tokens < 0 or not whole or num_tokens > self.lengths[src]
                or self.lengths[dst] != 0 or src == dst):
            raise InvalidArg("fork shares whole blocks, or all of the source, into an empty sequence")
        shared = self.tables[src][: blocks_for(num_tokens, bs)]
        for blk in shared:
            self.refcount[blk] += 1
        self.tables[dst] = list(shared)
        self.lengths[dst] = num_tokens

    def free_seq(self, seq: int) -> None:
        if seq not in self.tables:
            raise NotFound(seq)
        if seq in self.swapped:
            self.swapped.discard(seq)
            for blk in self.tables.pop(seq):
                self.host_refcount[blk] -= 1
                if self.host_refcount[blk] == 0:
                    self.host_free.append(blk)
        else:
            for blk in self.tables.pop(seq):
                self.refcount[blk] -= 1
                if self.refcount[blk] == 0:
                    self.free.append(blk)
        del self.lengths[seq]

    def _check_group(self, seqs: Sequence[int], want_swapped: bool) -> None:
        if self.num_host_blocks is None:
            raise InvalidArg("no host pool")
        if len(set(seqs)) != len(seqs):
            raise InvalidArg("a sequence is listed twice")
        for s in seqs:
            if s not in self.tables:
                raise NotFound(s)
            if (s in self.swapped) != want_swapped:
                raise Swapped(f"sequence {s} is in the wrong state for this swap")

    def swap_out(self, seqs: Sequence[int]) -> List[Tuple[int, int]]:
        """Move the sequences' blocks to the host pool; returns the
        (device block, host block) copies to make."""
        self._check_group(seqs, want_swapped=False)
        distinct = {blk for s in seqs for blk in self.tables[s]}
        if len(distinct) > len(self.host_free):
            raise OutOfBlocks(f"need {len(distinct)} host blocks, {len(self.host_free)} free")
        to_host: Dict[int, int] = {}
        pairs = []
        for s in seqs:
            new_table = []
            for blk in self.tables[s]:
                if blk not in to_host:
                    to_host[blk] = self.host_free.popleft()
                    pairs.append((blk, to_host[blk]))
                self.host_refcount[to_host[blk]] += 1
                self.refcount[blk] -= 1
                if self.refcount[blk] == 0:
                    self.free.append(blk)
                new_table.append(to_host[blk])
            self.tables[s] = new_table
            self.swapped.add(s)
        return pairs

    def swap_in(self, seqs: Sequence[int]) -> List[Tuple[int, int]]:
        """Move swapped-out sequences back to fresh device blocks; returns the
        (host block, device block) copies to make."""
        self._check_group(seqs, want_swapped=True)
        distinct = {blk for s in seqs for blk in self.tables[s]}
        if len(distinct) > len(self.free):
            raise OutOfBlocks(f"need {len(distinct)} device blocks, {len(self.free)} free")
        to_dev: Dict[int, int] = {}
        pairs = []
        for s in seqs:
            new_table = []
            for blk in self.tables[s]:
                if blk not in to_dev:
                    to_dev[blk] = self._take_free()
                    pairs.append((blk, to_dev[blk]))
                self.refcount[to_dev[blk]] += 1
                self.host_refcount[blk] -= 1
                if self.host_refcount[blk] == 0:
                    self.host_free.append(blk)
                new_table.append(to_dev[blk])
            self.tables[s] = new_table
            self.swapped.discard(s)
        return pairs

    def build_block_tables(self, seqs: Sequence[int], max_blocks: int,
                           pad: int = -1) -> Tuple[np.ndarray, np.ndarray]:
        tables = np.full((len(seqs), max_blocks), pad, dtype=np.int32)
        ctx = np.zeros(len(seqs), dtype=np.int32)
        for s in seqs:
            self._resident(s)
        for i, s in enumerate(seqs):
            t = self.table(s)
            if len(t) > max_blocks:
                raise InvalidArg(f"sequence {s} has {len(t)} blocks > {max_blocks}")
            tables[i, : len(t)] = t
            ctx[i] = self.lengths[s]
        return tables, ctx

    def shared_prefix_members(self, seqs: Sequence[int], prefix_tokens: int) -> List[int]:
        """Positions in ``seqs`` of the sequences that share a prefix: longer
        than ``prefix_tokens`` and holding the same physical blocks for its
        first ``prefix_tokens // block_size`` blocks ("What Is vLLM …",
        memory-sharing step).  Sequences are grouped by that block list; the
        largest group of at least two is returned (the first met on a tie),
        else an empty list."""
        if prefix_tokens <= 0 or prefix_tokens % self.block_size:
            raise InvalidArg("prefix_tokens must be a positive multiple of the block size")
        if len(set(seqs)) != len(seqs):
            raise InvalidArg("a sequence is listed twice")
        for s in seqs:
            self._resident(s)
        nb = prefix_tokens // self.block_size
        groups: Dict[tuple, List[int]] = {}
        for i, s in enumerate(seqs):
            if self.lengths[s] > prefix_tokens:
                groups.setdefault(tuple(self.tables[s][:nb]), []).append(i)
        best: List[int] = []
        for g in groups.values():  # insertion order: first met wins a tie
            if len(g) >= 2 and len(g) > len(best):
                best = g
        return best

    # -- replay of a workload's op list -------------------------------------
    def replay(self, ops: Iterable[tuple]) -> None:
        for op in ops:
            if op[0] == "add":
                self.add(op[1])
            elif op[0] == "append":
                self.append(op[1], op[2])
            elif op[0] == "fork":
                self.fork_prefix(op[1], op[2], op[3])
            elif op[0] == "append_cow":
                self.append_cow(op[1], op[2])
            elif op[0] == "swap_out":
                self.swap_out(list(op[1]))
            elif op[0] == "swap_in":
                self.swap_in(list(op[1]))
            else:
                raise InvalidArg(op)
