"""Oracle: paged decode attention in float64 (test infrastructure only).

What is computed (the plain definition; the GPU path must reach the same
values up to rounding):

* every new token attends to all earlier tokens of its sequence and to itself,
  with no window and no other mask ("vLLM in Production …", section "The KV
  Cache and the 60–80% Memory Tax");
* the keys and values of a sequence sit in fixed-size blocks anywhere in the
  pool; a per-sequence block table maps logical block ``t // block_size`` to a
  physical block, and the row inside it is ``t % block_size`` ("vLLM in
  Production …", section "PagedAttention — Virtual Memory for the KV Cache";
  "What Is vLLM …", section "How does PagedAttention work?", block-table
  step, its worked position lookup);
* the cache holds ``[num_blocks, block_size, num_kv_heads, head_dim]`` for K
  and the same for V; query head ``h`` reads kv head ``h // (Hq / Hkv)``;
* ``out[b, h] = softmax(scale · K_b q[b, h]) · V_b`` over the ``ctx_b`` gathered
  rows; a sequence with no context yields zeros.

bfloat16 inputs arrive as raw 16-bit patterns and are widened exactly (the
pattern is the top half of a float32).
"""
from __future__ import annotations

import numpy as np

__all__ = ["widen", "gather_sequence", "attend", "paged_decode", "paged_decode_one",
           "softmax_weights", "paged_prefill"]


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (``dtype`` "f32" or "bf16" bits)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def gather_sequence(cache: np.ndarray, table_row, ctx: int, block_size: int) -> np.ndarray:
    """Contiguous ``[ctx, Hkv, D]`` rows of one sequence, read through its table.

    Token ``t`` lives in physical block ``table_row[t // block_size]`` at row
    ``t % block_size``."""
    rows = [cache[int(table_row[t // block_size]), t % block_size] for t in range(ctx)]
    if not rows:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.stack(rows)


def softmax_weights(logits: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, shifted by the row maximum (exact in math)."""
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Single-query attention for one head: ``q [D]``, ``k, v [T, D]`` → ``[D]``."""
    if k.shape[0] == 0:
        return np.zeros(v.shape[1], dtype=np.float64)
    logits = scale * (k @ q)
    return softmax_weights(logits) @ v


def paged_decode_one(q_bh: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     table_row, ctx: int, kv_head: int, block_size: int,
                     scale: float) -> np.ndarray:
    """Output of one (sequence, query head): all arguments already float64."""
    k = gather_sequence(k_cache, table_row, ctx, block_size)
    v = gather_sequence(v_cache, table_row, ctx, block_size)
    if ctx == 0:
        return np.zeros(q_bh.shape[-1], dtype=np.float64)
    return attend(q_bh, k[:, kv_head, :], v[:, kv_head, :], scale)


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                 dtype: str = "f32") -> np.ndarray:
    """Paged decode attention for a batch.

    ``q [B, Hq, D]``, caches ``[N, bs, Hkv, D]`` (stored elements of ``dtype``),
    ``block_tables [B, max_blocks]`` (entries past a sequence's blocks are never
    read), ``context_lens [B]``.  Returns float64 ``[B, Hq, D]``."""
    qf = widen(q, dtype)
    B, Hq, D = qf.shape
    Hkv = k_cache.shape[2]
    bs = k_cache.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    group = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        ctx = int(context_lens[b])
        if ctx == 0:
            continue
        # gather the stored rows first, widen only what the sequence uses
        k = widen(gather_sequence(k_cache, block_tables[b], ctx, bs), dtype)
        v = widen(gather_sequence(v_cache, block_tables[b], ctx, bs), dtype)
        for h in range(Hq):
            g = h // group
            out[b, h] = attend(qf[b, h], k[:, g, :], v[:, g, :], scale)
    return out


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
                  dtype: str = "f32") -> np.ndarray:
    """Several new tokens per sequence (a prompt chunk) attend to the paged cache.

    Long prompts are processed in pieces so one large prefill does not stall
    the decoding sequences ("Serving models with vLLM", section "How it works:
    continuous batching", chunked prefill).  Sequence ``b`` owns query rows
    ``query_start[b] .. query_start[b+1]-1`` of ``q [T, Hq, D]``; its chunk of
    ``n_b`` tokens is the end of its context (their K/V already in the cache),
    so query ``i`` sits at position ``ctx_b - n_b + i`` and, like any token,
    attends to every earlier token and itself ("vLLM in Production …",
    section "The KV Cache and the 60–80% Memory Tax") — positions ``0 ..
    ctx_b - n_b + i``.  A query whose position is negative (a chunk longer
    than its context) gets zeros.  Returns float64 ``[T, Hq, D]``."""
    qf = widen(q, dtype)
    T, Hq, D = qf.shape
    Hkv = k_cache.shape[2]
    bs = k_cache.shape[1]
    group = Hq // Hkv
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for b in range(len(context_lens)):
        ctx = int(context_lens[b])
        lo, hi = int(query_start[b]), int(query_start[b + 1])
        n = hi - lo
        if ctx == 0 or n == 0:
            continue
        k = widen(gather_sequence(k_cache, block_tables[b], ctx, bs), dtype)
        v = widen(gather_sequence(v_cache, block_tables[b], ctx, bs), dtype)
        for i in range(n):
            pos = ctx - n + i
            if pos < 0:
                continue
            for h in range(Hq):
                g = h // group
                out[lo + i, h] = attend(qf[lo + i, h], k[: pos + 1, g, :], v[: pos + 1, g, :], scale)
    return out
