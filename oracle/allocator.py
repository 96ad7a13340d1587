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

Token ``pos`` of a sequence is stored at slot ``table[pos // bs] * bs + pos % bs``.
Test infrastructure only.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = ["AllocatorError", "OutOfBlocks", "NotFound", "SharedWrite", "InvalidArg",
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
        if seq not in self.tables:
            raise NotFound(seq)
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
                blk = self.free.popleft()
                self.refcount[blk] += 1
                table.append(blk)
            slots.append(slot_of(table, pos, bs))
        self.lengths[seq] = length + n
        return slots

    def append_cow(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Grow ``seq`` by ``n`` tokens, copying a shared, partly filled last
        block first.  Returns (slots, copy pairs (source block, new block))."""
        if seq not in self.tables:
            raise NotFound(seq)
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
            new = self.free.popleft()
            self.refcount[new] += 1
            self.refcount[old] -= 1
            table[-1] = new
            pairs.append((old, new))
        return self.append(seq, n), pairs

    def fork_prefix(self, src: int, dst: int, num_tokens: int) -> None:
        """Make ``dst`` (empty) share the first ``num_tokens`` tokens of ``src``."""
        if src not in self.tables or dst not in self.tables:
            raise NotFound((src, dst))
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
        for blk in self.tables.pop(seq):
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.free.append(blk)
        del self.lengths[seq]

    def build_block_tables(self, seqs: Sequence[int], max_blocks: int,
                           pad: int = -1) -> Tuple[np.ndarray, np.ndarray]:
        tables = np.full((len(seqs), max_blocks), pad, dtype=np.int32)
        ctx = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self.table(s)
            if len(t) > max_blocks:
                raise InvalidArg(f"sequence {s} has {len(t)} blocks > {max_blocks}")
            tables[i, : len(t)] = t
            ctx[i] = self.lengths[s]
        return tables, ctx

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
            else:
                raise InvalidArg(op)
