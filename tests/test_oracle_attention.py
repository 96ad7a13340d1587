"""Pins of the attention oracle against things other than itself.

Each ``pin_*`` function takes the oracle module as an argument so that
``test_oracle_mutations.py`` can run the same pins against deliberately broken
copies of the oracle and show that every planted mistake is caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle.attention as OA
import workloads as W

pytestmark = []


# ---------------------------------------------------------------- helpers
def _rand(seed, *shape):
    return W.normal_f32(seed, 7, int(np.prod(shape))).reshape(shape).astype(np.float64)


def _page(contig_k, contig_v, ctxs, bs, perm_seed, pad=-1, extra_blocks=3, poison=np.nan):
    """Scatter contiguous per-sequence K/V ``[B][T_b, Hkv, D]`` into a paged pool.

    Written independently of the oracle: the pool is filled block by block, with
    logical block j of sequence b placed at a seeded random physical block."""
    nbs = [-(-c // bs) for c in ctxs]
    total = sum(nbs) + extra_blocks
    perm = W.permutation(perm_seed, total)
    Hkv, D = contig_k[0].shape[1:]
    kc = np.full((total, bs, Hkv, D), poison)
    vc = np.full((total, bs, Hkv, D), poison)
    maxb = max(nbs + [1]) + 2
    tables = np.full((len(ctxs), maxb), pad, dtype=np.int64)
    nxt = 0
    for b, c in enumerate(ctxs):
        for j in range(nbs[b]):
            phys = int(perm[nxt]); nxt += 1
            tables[b, j] = phys
            lo, hi = j * bs, min(c, (j + 1) * bs)
            kc[phys, : hi - lo] = contig_k[b][lo:hi]
            vc[phys, : hi - lo] = contig_v[b][lo:hi]
    return kc, vc, tables


def _brute(q, contig_k, contig_v, scale, group):
    """Plain loops with math.exp, softmax written as exp(s_i) / sum_j exp(s_j)."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        T = contig_k[b].shape[0]
        for h in range(Hq):
            g = h // group
            s = [scale * sum(q[b, h, d] * contig_k[b][t, g, d] for d in range(D)) for t in range(T)]
            e = [math.exp(x) for x in s]
            z = sum(e)
            for d in range(D):
                out[b, h, d] = sum(e[t] * contig_v[b][t, g, d] for t in range(T)) / z if T else 0.0
    return out


def _case(seed, ctxs, Hq, Hkv, D, bs):
    q = _rand(seed, len(ctxs), Hq, D)
    ck = [_rand(seed + 11 + b, c, Hkv, D) for b, c in enumerate(ctxs)]
    cv = [_rand(seed + 57 + b, c, Hkv, D) for b, c in enumerate(ctxs)]
    return q, ck, cv


# ---------------------------------------------------------------- pins
def pin_brute_force(mod):
    """Paged oracle == unpaged brute force (every group size, block size, D)."""
    for (ctxs, Hq, Hkv, D, bs) in [([1, 5, 17], 2, 2, 4, 4), ([9, 33, 2], 4, 2, 8, 8),
                                     ([20, 7], 8, 1, 4, 16), ([40, 1, 16], 6, 3, 2, 32)]:
        q, ck, cv = _case(3, ctxs, Hq, Hkv, D, bs)
        kc, vc, tb = _page(ck, cv, ctxs, bs, perm_seed=sum(ctxs))
        got = mod.paged_decode(q.astype(np.float32), kc.astype(np.float32), vc.astype(np.float32),
                               tb, np.array(ctxs), 0.37, "f32")
        ref = _brute(q.astype(np.float32).astype(np.float64), [k.astype(np.float32).astype(np.float64) for k in ck],
                     [v.astype(np.float32).astype(np.float64) for v in cv], 0.37, Hq // Hkv)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def pin_torch_sdpa(mod):
    """Contiguous special case == torch's scaled_dot_product_attention in float64."""
    ctxs, Hq, Hkv, D, bs = [23, 64, 3], 8, 2, 16, 16
    q, ck, cv = _case(5, ctxs, Hq, Hkv, D, bs)
    kc, vc, tb = _page(ck, cv, ctxs, bs, perm_seed=99)
    got = mod.paged_decode(q.astype(np.float32), kc.astype(np.float32), vc.astype(np.float32),
                           tb, np.array(ctxs), 0.25, "f32")
    for b, c in enumerate(ctxs):
        qt = torch.from_numpy(q[b].astype(np.float32).astype(np.float64))[:, None, :]  # [Hq,1,D]
        kt = torch.from_numpy(ck[b].astype(np.float32).astype(np.float64)).permute(1, 0, 2)  # [Hkv,T,D]
        vt = torch.from_numpy(cv[b].astype(np.float32).astype(np.float64)).permute(1, 0, 2)
        kt = kt.repeat_interleave(Hq // Hkv, dim=0)
        vt = vt.repeat_interleave(Hq // Hkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.25)[:, 0, :]
        np.testing.assert_allclose(got[b], ref.numpy(), rtol=1e-12, atol=1e-13)


def pin_closed_forms(mod):
    D = 8
    rng_v = _rand(21, 7, D)
    q = _rand(22, D)
    # all keys equal -> mean of V
    k = np.tile(_rand(23, 1, D), (7, 1))
    np.testing.assert_allclose(mod.attend(q, k, rng_v, 0.7), rng_v.mean(0), rtol=1e-13, atol=1e-14)
    # scale 0 -> mean of V
    np.testing.assert_allclose(mod.attend(q, _rand(24, 7, D), rng_v, 0.0), rng_v.mean(0), rtol=1e-13, atol=1e-14)
    # one context token -> that value row
    np.testing.assert_allclose(mod.attend(q, _rand(25, 1, D), rng_v[:1], 0.9), rng_v[0], rtol=1e-14)
    # two tokens -> logistic weights
    k2 = _rand(26, 2, D)
    s0, s1 = 0.9 * k2[0] @ q, 0.9 * k2[1] @ q
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    ref = sig(s0 - s1) * rng_v[0] + sig(s1 - s0) * rng_v[1]
    np.testing.assert_allclose(mod.attend(q, k2, rng_v[:2], 0.9), ref, rtol=1e-12, atol=1e-14)
    # one logit far above the rest -> that row
    k3 = _rand(27, 7, D) * 0.01
    k3[4] = q * (1e3 / (q @ q))
    np.testing.assert_allclose(mod.attend(q, k3, rng_v, 1.0), rng_v[4], rtol=1e-12, atol=1e-12)
    # weights are a distribution
    w = mod.softmax_weights(np.array([[3.0, -1.0, 0.5, 700.0], [1e-3, 2e-3, 0, 0]]))
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=0, atol=1e-15)
    assert (w >= 0).all()
    # the softmax itself: exp(s_i)/sum exp(s_j) on small logits
    s = np.array([0.3, -1.2, 2.0])
    e = np.exp(s)
    np.testing.assert_allclose(mod.softmax_weights(s[None])[0], e / e.sum(), rtol=1e-15)


def pin_widen(mod):
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x8000], dtype=np.uint16)
    got = mod.widen(bits, "bf16")
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 1.0 + 2.0 ** -7
    assert got[3] == 2.0 ** -133 and np.isinf(got[4]) and got[5] == 0.0
    assert np.signbit(got[5])
    f = np.array([1.5, -3.25e-3], dtype=np.float32)
    assert (mod.widen(f, "f32") == f.astype(np.float64)).all()


def pin_placement_and_sharing(mod):
    """Output is the same for any physical placement and for shared vs copied prefix blocks."""
    ctxs, Hq, Hkv, D, bs = [37, 50, 16], 4, 2, 8, 16
    q, ck, cv = _case(31, ctxs, Hq, Hkv, D, bs)
    outs = []
    for seed in (1, 2, 3):
        kc, vc, tb = _page(ck, cv, ctxs, bs, perm_seed=seed)
        outs.append(mod.paged_decode(q, kc, vc, tb, np.array(ctxs), 0.3, "f32"))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    # sequences 0 and 1 share their first 32 tokens: duplicated vs shared blocks
    ck[1][:32] = ck[0][:32]
    cv[1][:32] = cv[0][:32]
    kc, vc, tb = _page(ck, cv, ctxs, bs, perm_seed=4)
    dup = mod.paged_decode(q, kc, vc, tb, np.array(ctxs), 0.3, "f32")
    tb2 = tb.copy()
    tb2[1, :2] = tb[0, :2]
    shared = mod.paged_decode(q, kc, vc, tb2, np.array(ctxs), 0.3, "f32")
    assert np.array_equal(dup, shared)


def pin_unused_slots_and_padding(mod):
    """Slots past the context and table entries past the last block are never read."""
    ctxs, Hq, Hkv, D, bs = [5, 17, 0], 2, 2, 4, 16
    q, ck, cv = _case(41, ctxs, Hq, Hkv, D, bs)
    kc, vc, tb = _page(ck, cv, ctxs, bs, perm_seed=5, pad=10 ** 9, poison=np.nan)
    out = mod.paged_decode(q, kc, vc, tb, np.array(ctxs), 0.5, "f32")
    assert np.isfinite(out).all()
    assert (out[2] == 0).all()
    ref = _brute(q.astype(np.float32).astype(np.float64), ck, cv, 0.5, 1)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def pin_one(mod):
    """The one-output entry point agrees with brute force for a GQA head."""
    ctxs, Hq, Hkv, D, bs = [29], 4, 2, 8, 8
    q, ck, cv = _case(51, ctxs, Hq, Hkv, D, bs)
    kc, vc, tb = _page(ck, cv, ctxs, bs, perm_seed=6)
    ref = _brute(q, ck, cv, 0.3, 2)
    for h in range(Hq):
        got = mod.paged_decode_one(q[0, h], kc, vc, tb[0], 29, h // 2, bs, 0.3)
        np.testing.assert_allclose(got, ref[0, h], rtol=1e-12, atol=1e-13)
    # no context: zeros, whatever the table holds
    assert (mod.paged_decode_one(q[0, 0], kc, vc, [10 ** 9], 0, 0, bs, 0.3) == 0).all()
    assert (mod.attend(q[0, 0], np.zeros((0, D)), np.zeros((0, D)), 0.3) == 0).all()


def _brute_causal(q_rows, contig_k, contig_v, ctxs, starts, scale, group):
    """Loops with math.exp; query i of sequence b sees tokens 0..ctx-n+i."""
    T, Hq, D = q_rows.shape
    out = np.zeros((T, Hq, D))
    for b, c in enumerate(ctxs):
        lo, hi = starts[b], starts[b + 1]
        n = hi - lo
        for i in range(n):
            pos = c - n + i
            if pos < 0:
                continue
            for h in range(Hq):
                g = h // group
                e = [math.exp(scale * sum(q_rows[lo + i, h, d] * contig_k[b][t, g, d] for d in range(D)))
                     for t in range(pos + 1)]
                z = sum(e)
                for d in range(D):
                    out[lo + i, h, d] = sum(e[t] * contig_v[b][t, g, d] for t in range(pos + 1)) / z
    return out


def pin_prefill(mod):
    """Chunked prefill: brute-force causal loops, torch SDPA with an explicit
    bottom-right causal mask, and the one-query case equal to decode."""
    ctxs, Hq, Hkv, D, bs = [9, 20, 4, 17], 4, 2, 4, 8
    chunks = [3, 20, 6, 1]          # the third chunk is longer than its context
    starts = np.concatenate([[0], np.cumsum(chunks)])
    q = _rand(61, int(starts[-1]), Hq, D)
    _, ck, cv = _case(62, ctxs, Hq, Hkv, D, bs)
    kc, vc, tb = _page(ck, cv, ctxs, bs, perm_seed=8)
    got = mod.paged_prefill(q, kc, vc, tb, np.array(ctxs), starts, 0.41, "f32")
    ref = _brute_causal(q, ck, cv, ctxs, starts, 0.41, Hq // Hkv)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    assert (got[starts[2]:starts[2] + 2] == 0).all()  # positions -2, -1
    b = 1
    qt = torch.from_numpy(q[starts[b]:starts[b + 1]]).permute(1, 0, 2)              # [Hq, n, D]
    kt = torch.from_numpy(ck[b]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)  # [Hq, T, D]
    vt = torch.from_numpy(cv[b]).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    n, T = chunks[b], ctxs[b]
    mask = torch.tensor([[t <= T - n + i for t in range(T)] for i in range(n)])
    sd = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.41)
    np.testing.assert_allclose(got[starts[b]:starts[b + 1]], sd.permute(1, 0, 2).numpy(),
                               rtol=1e-12, atol=1e-13)
    # one query per sequence is the decode step
    ones = np.arange(len(ctxs) + 1)
    q1 = _rand(63, len(ctxs), Hq, D)
    np.testing.assert_allclose(mod.paged_prefill(q1, kc, vc, tb, np.array(ctxs), ones, 0.41, "f32"),
                               mod.paged_decode(q1, kc, vc, tb, np.array(ctxs), 0.41, "f32"),
                               rtol=1e-15, atol=0)


PINS = [pin_brute_force, pin_torch_sdpa, pin_closed_forms, pin_widen,
        pin_placement_and_sharing, pin_unused_slots_and_padding, pin_one, pin_prefill]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_attention_oracle(pin):
    pin(OA)


def test_bytes_per_token_closed_form():
    """LLaMA-13B at fp16 keeps up to about 1.7 GB of KV per sequence ("vLLM in
    Production …", section on the KV cache).  With the public LLaMA-13B shape
    (40 layers, 40 heads of 128, 2048 tokens) the per-token K+V bytes are
    2·40·40·128·2 = 819,200 and a full sequence holds 1.68 GB."""
    per_layer = W.shape(2)  # 40 heads of 128, bf16 (2 bytes like fp16)
    per_token_layer = 2 * per_layer.num_kv_heads * per_layer.head_dim * per_layer.elem_bytes
    per_token = per_token_layer * 40
    assert per_token == 819_200
    assert abs(per_token * 2048 / 1e9 - 1.7) < 0.05
