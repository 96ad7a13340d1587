"""Oracle: writing new tokens' keys and values into the paged cache.

A sequence grows one token at a time; each new token's K and V rows go to the
slot the allocator handed out for its position, i.e. row ``slot % block_size``
of physical block ``slot // block_size`` ("vLLM in Production …", section
"PagedAttention — Virtual Memory for the KV Cache": blocks are filled as
tokens arrive).  A negative slot marks a padding token that is not written.
Every other byte of the cache is left as it was.  Test infrastructure only.
"""
from __future__ import annotations

import numpy as np

__all__ = ["reshape_and_cache"]


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
