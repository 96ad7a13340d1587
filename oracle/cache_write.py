"""Oracle: writing new tokens' keys and values into the paged cache.

A sequence grows one token at a time; each new token's K and V rows go to the
slot the allocator handed out for its position, i.e. row ``slot % block_size``
of physical block ``slot // block_size`` ("vLLM in Production …", section
"PagedAttention — Virtual Memory for the KV Cache": blocks are filled as
tokens arrive).  A negative slot marks a padding token that is not written.
Every other byte of the cache is left as it was.

Swapping a preempted sequence moves its blocks whole between the device cache
and a cache pool in host memory ("What Is vLLM …", section "What is
continuous batching in vLLM?", step 2): ``move_blocks`` is that copy, block
``dst`` of the target pool becoming block ``src`` of the source pool for each
(src, dst) pair.  Test infrastructure only.
"""
from __future__ import annotations

import numpy as np

__all__ = ["reshape_and_cache", "move_blocks"]


def reshape_and_cache(key: np.ndarray, value: np.ndarray, k_cache: np.ndarray,
                      v_cache: np.ndarray, slot_mapping) -> tuple:
    """Return copies of the caches with token ``i`` stored at ``slot_mapping[i]``.

    ``key, value [T, Hkv, D]``; caches ``[N, bs, Hkv, D]`` of the same element
    type (copied bit for bit)."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    bs = k_cache.shape[1]
    for i, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        kc[slot // bs, slot % bs] = key[i]
        vc[slot // bs, slot % bs] = value[i]
    return kc, vc


def move_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                pairs) -> tuple:
    """Return copies of the target pools ``dst_k, dst_v [M, bs, Hkv, D]`` in
    which block ``d`` holds block ``s`` of ``src_k, src_v [N, bs, Hkv, D]``
    for each pair ``(s, d)``; every other block is left as it was."""
    k = dst_k.copy()
    v = dst_v.copy()
    for s, d in pairs:
        k[int(d)] = src_k[int(s)]
        v[int(d)] = src_v[int(s)]
    return k, v
