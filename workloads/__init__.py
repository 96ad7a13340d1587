"""Seeded synthetic decode workloads for PagedAttention.

This module only draws inputs: context lengths, the order in which the pool
hands out free blocks, which sequences share a prompt prefix, the random
q / K / V payloads and the new tokens written each decode step.  It holds none
of the method's arithmetic (no block tables, no slots, no attention): the
block allocator and the attention are computed separately by the product
library and by the CPU oracle, and both read the same inputs from here.

Recipes (numpy PCG64, seed 1000 + config index unless stated):

* payloads are N(0, 1) fp32; bf16 workloads round them to bf16 with
  round-to-nearest-even and hand out the raw 16-bit patterns (``uint16``);
* context lengths follow the five decode shapes below; the log-normal mix uses
  median 600 and sigma 1.0 in natural-log space, rounded then clipped;
* the physical placement comes from ``free_order``, a seeded permutation of
  the pool ids that the allocator hands out first-in first-out;
* the prefix-sharing shape draws 128 sharers among sequences longer than the
  1024-token prefix.

Large payloads are drawn in fixed chunks, each from its own
``SeedSequence([seed, stream, chunk])``, so results do not depend on the
number of worker threads.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "DecodeShape",
    "SHAPES",
    "shape",
    "Workload",
    "make_workload",
    "normal_f32",
    "f32_to_bf16_bits",
    "normal_bf16_bits",
    "BF16_NAN_BITS",
]

BF16_NAN_BITS = np.uint16(0x7FC0)
_CHUNK = 1 << 22  # elements per independently seeded chunk

# stream ids for SeedSequence: one per kind of payload
_S_Q, _S_K, _S_V, _S_NEWK, _S_NEWV, _S_PERM, _S_CTX, _S_SHARE = range(8)


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    """One synthetic decode batch (one attention layer, one query per sequence)."""

    name: str
    dtype: str                 # "f32" or "bf16"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    ctx_kind: str              # "fixed" | "uniform" | "lognormal"
    ctx_fixed: Tuple[int, ...] = ()
    ctx_lo: int = 0
    ctx_hi: int = 0
    ctx_median: float = 0.0
    ctx_sigma: float = 0.0
    pool_blocks: Optional[int] = None   # None: sized to exactly fit the batch
    new_tokens: bool = False            # one new token per sequence written each step
    shared_prefix_tokens: int = 0
    num_sharers: int = 0
    partition_size: int = 0             # 0: single pass over each sequence
    chunk: int = 0                      # > 0: a prefill step of this many new tokens per sequence
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


SHAPES: Tuple[DecodeShape, ...] = (
    DecodeShape("tiny_fp32", "f32", 4, 4, 4, 64, 16, "fixed", ctx_fixed=(5, 17, 33, 100),
                pool_blocks=64, seed=1000),
    DecodeShape("llama7b_bf16", "bf16", 64, 32, 32, 128, 16, "uniform", ctx_lo=128,
                ctx_hi=2048, seed=1001),
    DecodeShape("llama13b_bf16", "bf16", 128, 40, 40, 128, 16, "lognormal",
                ctx_lo=16, ctx_hi=4096, ctx_median=600.0, ctx_sigma=1.0,
                new_tokens=True, seed=1002),
    DecodeShape("gqa_prefix_bf16", "bf16", 256, 32, 8, 128, 32, "uniform", ctx_lo=512,
                ctx_hi=8192, shared_prefix_tokens=1024, num_sharers=128, seed=1003),
    DecodeShape("long_splitk_bf16", "bf16", 32, 64, 8, 128, 16, "uniform", ctx_lo=16384,
                ctx_hi=32768, partition_size=512, seed=1004),
    # chunked prefill (not one of the five decode shapes): 16 LLaMA-13B-shaped
    # sequences each add a 512-token prompt chunk after 0..3584 earlier tokens
    DecodeShape("prefill_chunk_bf16", "bf16", 16, 40, 40, 128, 16, "uniform", ctx_lo=512,
                ctx_hi=4096, chunk=512, seed=1005),
)


def shape(index: int, **overrides) -> DecodeShape:
    """The decode shape ``index`` (0..4), optionally with fields replaced."""
    s = SHAPES[index]
    return dataclasses.replace(s, **overrides) if overrides else s


def _rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, chunk])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, stream: int, count: int) -> np.ndarray:
    """``count`` N(0,1) float32 values, chunk-seeded (thread-count independent)."""
    out = np.empty(count, dtype=np.float32)
    nchunks = (count + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        lo = c * _CHUNK
        hi = min(count, lo + _CHUNK)
        out[lo:hi] = _rng(seed, stream, c).standard_normal(hi - lo, dtype=np.float32)

    if nchunks <= 1:
        if count:
            fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def normal_bf16_bits(seed: int, stream: int, count: int) -> np.ndarray:
    """The values of ``normal_f32(seed, stream, count)`` rounded to bf16 bits,
    drawn and rounded chunk by chunk (no float32 copy of the whole array)."""
    out = np.empty(count, dtype=np.uint16)
    nchunks = (count + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        lo = c * _CHUNK
        hi = min(count, lo + _CHUNK)
        out[lo:hi] = f32_to_bf16_bits(
            _rng(seed, stream, c).standard_normal(hi - lo, dtype=np.float32))

    if nchunks <= 1:
        if count:
            fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the raw bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = BF16_NAN_BITS
    return r


def _payload(s: DecodeShape, stream: int, shp: Tuple[int, ...]) -> np.ndarray:
    n = int(np.prod(shp)) if shp else 1
    if s.dtype == "f32":
        return normal_f32(s.seed, stream, n).reshape(shp)
    return normal_bf16_bits(s.seed, stream, n).reshape(shp)


def context_lens(s: DecodeShape) -> np.ndarray:
    """Per-sequence context lengths (tokens attended, the new token included)."""
    g = _rng(s.seed, _S_CTX)
    if s.ctx_kind == "fixed":
        ctx = np.array(s.ctx_fixed, dtype=np.int64)
        assert len(ctx) == s.num_seqs
    elif s.ctx_kind == "uniform":
        ctx = g.integers(s.ctx_lo, s.ctx_hi, size=s.num_seqs, endpoint=True)
    elif s.ctx_kind == "lognormal":
        x = g.lognormal(mean=math.log(s.ctx_median), sigma=s.ctx_sigma, size=s.num_seqs)
        ctx = np.clip(np.rint(x), s.ctx_lo, s.ctx_hi).astype(np.int64)
    else:  # pragma: no cover
        raise ValueError(s.ctx_kind)
    return ctx.astype(np.int64)


def sharers(s: DecodeShape, ctx: np.ndarray) -> np.ndarray:
    """Indices of the sequences that share the common prefix (sorted ascending).

    Sharers are drawn among sequences with at least one private token after
    the prefix, so every sharer owns private blocks too."""
    if not s.num_sharers:
        return np.zeros(0, dtype=np.int64)
    eligible = np.nonzero(ctx > s.shared_prefix_tokens)[0]
    if len(eligible) < s.num_sharers:
        raise ValueError("not enough sequences longer than the shared prefix")
    pick = _rng(s.seed, _S_SHARE).choice(eligible, size=s.num_sharers, replace=False)
    return np.sort(pick).astype(np.int64)


@dataclasses.dataclass
class Workload:
    """Inputs of one synthetic decode step.

    ``ops`` is the order in which sequences are created and grown; both block
    allocators replay it.  Each op is one of
    ``("add", seq)``, ``("append", seq, n_tokens)``,
    ``("fork", src_seq, dst_seq, n_tokens)``.
    After ``ops``, a step with ``new_tokens`` appends one token per sequence
    (in sequence order) and writes ``new_k`` / ``new_v`` through the slots; a
    prefill shape (``chunk`` > 0) appends ``chunk`` tokens per sequence, whose
    ``q`` rows are ``[B * chunk, Hq, D]`` in sequence order.
    """

    shape: DecodeShape
    ctx: np.ndarray             # int64 [B], context after the step
    sharers: np.ndarray         # int64 [num_sharers]
    num_blocks: int
    free_order: np.ndarray      # int32 [num_blocks] permutation
    ops: List[tuple]
    q: np.ndarray               # [B, Hq, D]  f32 or bf16 bits
    k_cache: np.ndarray         # [N, bs, Hkv, D]
    v_cache: np.ndarray
    new_k: Optional[np.ndarray]  # [B, Hkv, D] or None
    new_v: Optional[np.ndarray]

    @property
    def kv_bytes(self) -> int:
        s = self.shape
        return int(self.ctx.sum()) * 2 * s.num_kv_heads * s.head_dim * s.elem_bytes


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def pool_blocks_needed(s: DecodeShape, ctx: np.ndarray, shared: np.ndarray,
                       extra_tokens: int = 0) -> int:
    """Pool size that exactly fits the batch (shared prefix blocks counted once).

    ``extra_tokens`` reserves room for that many further tokens per sequence."""
    bs = s.block_size
    pre = s.shared_prefix_tokens // bs if len(shared) else 0
    total = 0
    is_sharer = np.zeros(len(ctx), dtype=bool)
    is_sharer[shared] = True
    for b, c in enumerate(ctx):
        nb = _ceil_div(int(c) + extra_tokens, bs)
        total += nb - pre if is_sharer[b] else nb
    return total + pre


def make_workload(s: DecodeShape, with_payload: bool = True,
                  extra_tokens: int = 0) -> Workload:
    """Draw the inputs of one decode step of shape ``s``.

    ``extra_tokens`` enlarges the pool so that each sequence can later grow by
    that many tokens (used by repeated decode steps)."""
    ctx = context_lens(s)
    shared = sharers(s, ctx)
    if s.pool_blocks is not None:
        n_blocks = s.pool_blocks
    else:
        n_blocks = pool_blocks_needed(s, ctx, shared, extra_tokens)
    free_order = _rng(s.seed, _S_PERM).permutation(n_blocks).astype(np.int32)

    ops: List[tuple] = []
    pre = s.shared_prefix_tokens
    for b in range(s.num_seqs):
        ops.append(("add", b))
    if len(shared):
        first = int(shared[0])
        ops.append(("append", first, pre))
        for b in shared[1:]:
            ops.append(("fork", first, int(b), pre))
    is_sharer = set(int(b) for b in shared)
    step_tokens_ = s.chunk if s.chunk else (1 if s.new_tokens else 0)
    for b in range(s.num_seqs):
        n = int(ctx[b]) - (pre if b in is_sharer else 0) - step_tokens_
        if n > 0:
            ops.append(("append", b, n))

    B, Hq, Hkv, D, bs = s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim, s.block_size
    q = k_cache = v_cache = new_k = new_v = None
    if with_payload:
        rows = B * s.chunk if s.chunk else B
        q = _payload(s, _S_Q, (rows, Hq, D))
        k_cache = _payload(s, _S_K, (n_blocks, bs, Hkv, D))
        v_cache = _payload(s, _S_V, (n_blocks, bs, Hkv, D))
        if s.new_tokens or s.chunk:
            new_k = _payload(s, _S_NEWK, (rows, Hkv, D))
            new_v = _payload(s, _S_NEWV, (rows, Hkv, D))
    return Workload(s, ctx, shared, n_blocks, free_order, ops, q, k_cache, v_cache, new_k, new_v)


def step_tokens(s: DecodeShape, step: int) -> Tuple[np.ndarray, np.ndarray]:
    """New K/V rows ``[B (x chunk), Hkv, D]`` for a later step ``step`` >= 1."""
    shp = (s.num_seqs * (s.chunk or 1), s.num_kv_heads, s.head_dim)
    return (_payload(dataclasses.replace(s, seed=s.seed * 1000 + step), _S_NEWK, shp),
            _payload(dataclasses.replace(s, seed=s.seed * 1000 + step), _S_NEWV, shp))


def permutation(seed: int, n: int) -> np.ndarray:
    """A seeded permutation of ``0..n-1`` (for placement-invariance checks)."""
    return _rng(seed, _S_PERM, 1).permutation(n).astype(np.int64)


def random_lengths(seed: int, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` seeded integers in ``[lo, hi]`` (for property checks)."""
    return _rng(seed, _S_CTX, 1).integers(lo, hi, size=count, endpoint=True).astype(np.int64)


def scaled(s: DecodeShape, num_seqs: int, ctx_hi: Optional[int] = None,
           ctx_lo: Optional[int] = None, num_sharers: Optional[int] = None) -> DecodeShape:
    """A smaller copy of ``s`` with the same structure, for checks the oracle
    runs in seconds."""
    kw = {"num_seqs": num_seqs}
    if ctx_hi is not None:
        kw["ctx_hi"] = ctx_hi
    if ctx_lo is not None:
        kw["ctx_lo"] = ctx_lo
    if num_sharers is not None:
        kw["num_sharers"] = num_sharers
    if s.ctx_kind == "fixed":
        kw["ctx_fixed"] = tuple(s.ctx_fixed[:num_seqs])
    return dataclasses.replace(s, **kw)
