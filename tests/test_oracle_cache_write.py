"""Pins of the cache-write oracle: a round trip through the slots, bytes off the
slots untouched, padding slots skipped."""
import numpy as np

import oracle.cache_write as OC
import workloads as W


def pin_round_trip(mod):
    N, bs, Hkv, D, T = 6, 4, 3, 8, 9
    kc = W.f32_to_bf16_bits(W.normal_f32(1, 1, N * bs * Hkv * D)).reshape(N, bs, Hkv, D)
    vc = W.f32_to_bf16_bits(W.normal_f32(1, 2, N * bs * Hkv * D)).reshape(N, bs, Hkv, D)
    key = W.f32_to_bf16_bits(W.normal_f32(1, 3, T * Hkv * D)).reshape(T, Hkv, D)
    val = W.f32_to_bf16_bits(W.normal_f32(1, 4, T * Hkv * D)).reshape(T, Hkv, D)
    slots = W.permutation(11, N * bs)[:T].copy()
    slots[3] = -1  # a padding token
    k2, v2 = mod.reshape_and_cache(key, val, kc, vc, slots)
    flat_k = k2.reshape(N * bs, Hkv, D)
    flat_v = v2.reshape(N * bs, Hkv, D)
    touched = np.zeros(N * bs, dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        touched[s] = True
        assert np.array_equal(flat_k[s], key[i]) and np.array_equal(flat_v[s], val[i])
    assert np.array_equal(flat_k[~touched], kc.reshape(N * bs, Hkv, D)[~touched])
    assert np.array_equal(flat_v[~touched], vc.reshape(N * bs, Hkv, D)[~touched])
    assert touched.sum() == T - 1
    # the inputs are not modified
    assert not np.shares_memory(k2, kc)


PINS = [pin_round_trip]


def test_cache_write_oracle():
    for p in PINS:
        p(OC)
