"""The fused decode step (cache write + attention in one launch) against the
oracle doing the two steps in order ("vLLM in Production …", section
"PagedAttention — Virtual Memory for the KV Cache": the new token's K/V go
into its slot, and the token attends to its whole context, itself included).

Each case replays a workload on both allocators, appends one token per
sequence, then runs pkv_paged_attention_decode_write on caches that do not
yet hold the new rows.  The caches must equal the oracle's cache write bit
for bit, and the output must be within the tolerance of the oracle decode and
of the product's own separate cache write + decode (the fused kernel adds the
new token after the cached ones, so the rounding order differs)."""
import dataclasses

import numpy as np
import pytest

import oracle.allocator as OAL
import oracle.attention as OA
import oracle.cache_write as OC
import workloads as W
from gpu_cases import assert_close, from_dev, log, poison_unused_tail, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)
import paged_kv_cache_292_amd as P  # noqa: E402


@pytest.fixture
def decode_path():
    """Select a decode kernel for one test, restore the automatic choice after."""
    yield P.set_decode_path
    P.set_decode_path(P.PATH_AUTO)


def _with_new(s):
    return dataclasses.replace(s, new_tokens=True)


CASES = {
    "tiny_fp32": _with_new(W.shape(0)),
    "llama7b": _with_new(W.scaled(W.shape(1), num_seqs=6)),
    "llama13b": W.scaled(W.shape(2), num_seqs=12),
    "gqa_prefix": _with_new(W.scaled(W.shape(3), num_seqs=16, num_sharers=6)),
    "long_splitk": _with_new(W.scaled(W.shape(4), num_seqs=3)),
    "groups_g2_hkv3": W.DecodeShape("g2", "bf16", 5, 6, 3, 128, 16, "fixed",
                                    ctx_fixed=(1, 17, 200, 33, 512), new_tokens=True, seed=41),
    "groups_g8_d64": W.DecodeShape("g8", "bf16", 4, 16, 2, 64, 32, "fixed",
                                   ctx_fixed=(1, 31, 96, 700), new_tokens=True, seed=42),
    "f32_g2_d128": W.DecodeShape("f32g2", "f32", 4, 8, 4, 128, 32, "fixed",
                                 ctx_fixed=(2, 65, 300, 33), new_tokens=True, seed=43),
}


def _setup(s):
    wl = W.make_workload(s)
    B = s.num_seqs
    o = OAL.BlockAllocator(wl.num_blocks, s.block_size, wl.free_order)
    o.replay(wl.ops)
    p = P.Allocator(wl.num_blocks, s.block_size, wl.free_order)
    p.replay(wl.ops)
    so = np.array([o.append(b, 1)[0] for b in range(B)], dtype=np.int64)
    sp = p.append_tokens(list(range(B)), [1] * B)
    assert np.array_equal(so, sp)
    mb = max(len(o.tables[b]) for b in range(B)) + 2
    tables, ctx = o.build_block_tables(list(range(B)), mb, pad=-1)
    tp, cp = p.build_block_tables(list(range(B)), mb, pad=-1)
    assert np.array_equal(tables, tp) and np.array_equal(ctx, cp)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    poison_unused_tail(kc, tables, ctx, s.dtype)
    poison_unused_tail(vc, tables, ctx, s.dtype)
    nan = np.float32(np.nan) if s.dtype == "f32" else W.BF16_NAN_BITS
    for sl in so:  # the new slots hold garbage until written
        kc[sl // s.block_size, sl % s.block_size] = nan
        vc[sl // s.block_size, sl % s.block_size] = nan
    return wl, so, tables, ctx, kc, vc


def _bits(a: np.ndarray) -> np.ndarray:
    """Stored bit patterns (the poisoned slots hold NaN, which != itself)."""
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _run(s, wl, tables, ctx, kc, vc, part, fused, order=None):
    kd, vd = to_dev(kc, s.dtype), to_dev(vc, s.dtype)
    q = to_dev(wl.q, s.dtype)
    nk, nv = to_dev(wl.new_k, s.dtype), to_dev(wl.new_v, s.dtype)
    out = torch.empty_like(q)
    mx = int(ctx.max())
    wsb = P.decode_workspace_bytes(s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                   s.block_size, mx, part, P.F32 if s.dtype == "f32" else P.BF16)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    td, cd = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    so = torch.from_numpy(order).cuda() if order is not None else None
    if fused:
        P.paged_attention_decode_write(out, q, nk, nv, kd, vd, td, cd, mx, s.scale, part, ws,
                                       seq_order=so)
    else:
        slots = np.array([tables[b, (c - 1) // s.block_size] * s.block_size + (c - 1) % s.block_size
                          for b, c in enumerate(ctx)], dtype=np.int64)
        P.kv_reshape_and_cache(nk, nv, kd, vd, torch.from_numpy(slots).cuda())
        P.paged_attention_decode(out, q, kd, vd, td, cd, mx, s.scale, part, ws, seq_order=so)
    torch.cuda.synchronize()
    return from_dev(out, s.dtype), from_dev(kd, s.dtype), from_dev(vd, s.dtype)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("part", [0, 64, P.PARTITION_AUTO])
def test_fused_write_decode_matches_oracle(name, part, decode_path):
    s = CASES[name]
    wl, slots, tables, ctx, kc, vc = _setup(s)
    ko, vo = OC.reshape_and_cache(wl.new_k, wl.new_v, kc, vc, slots)
    ref = OA.paged_decode(wl.q, ko, vo, tables, ctx, s.scale, s.dtype)
    paths = [P.PATH_AUTO] if s.dtype == "f32" else [P.PATH_VALU, P.PATH_MFMA]
    for path in paths:
        decode_path(path)
        log(f"fused write+decode {name} partition={part} path={path}")
        got, kd, vd = _run(s, wl, tables, ctx, kc, vc, part, True)
        assert np.array_equal(_bits(kd), _bits(ko)) and np.array_equal(_bits(vd), _bits(vo)), \
            "cache after the fused write"
        assert_close(OA.widen(got, s.dtype), ref, s.dtype, f"fused {name} p{part} path{path}")
        sep, _, _ = _run(s, wl, tables, ctx, kc, vc, part, False)
        assert_close(OA.widen(got, s.dtype), OA.widen(sep, s.dtype), s.dtype,
                     f"fused vs separate {name} p{part} path{path}")


def test_fused_write_zero_context_and_launch_order(decode_path):
    """A sequence with no context writes nothing and outputs zeros; a launch
    order does not change anything."""
    s = CASES["groups_g2_hkv3"]
    wl, slots, tables, ctx, kc, vc = _setup(s)
    ctx0 = ctx.copy()
    ctx0[2] = 0  # sequence 2: no token at all this call
    keep = [i for i in range(s.num_seqs) if i != 2]
    ko, vo = OC.reshape_and_cache(wl.new_k[keep], wl.new_v[keep], kc, vc, slots[keep])
    ref = OA.paged_decode(wl.q, ko, vo, tables, ctx0, s.scale, s.dtype)
    order = P.longest_first_order(ctx0)
    got, kd, vd = _run(s, wl, tables, ctx0, kc, vc, 0, True, order=order)
    assert np.array_equal(_bits(kd), _bits(ko)) and np.array_equal(_bits(vd), _bits(vo))
    assert (OA.widen(got, s.dtype)[2] == 0).all()
    assert_close(OA.widen(got, s.dtype), ref, s.dtype, "fused, zero context, ordered")


def _run_step(s, wl, tables, ctx, kc, vc, part, nbytes, seed, order=None, rows=True):
    """pkv_paged_attention_decode_step with a seeded pinned source of nbytes
    (rows=False: a step without new tokens, both new-row arguments None)."""
    kd, vd = to_dev(kc, s.dtype), to_dev(vc, s.dtype)
    q = to_dev(wl.q, s.dtype)
    nk, nv = (to_dev(wl.new_k, s.dtype), to_dev(wl.new_v, s.dtype)) if rows else (None, None)
    out = torch.empty_like(q)
    mx = int(ctx.max())
    wsb = P.decode_workspace_bytes(s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                   s.block_size, mx, part, P.F32 if s.dtype == "f32" else P.BF16)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
    src_np = np.random.default_rng(seed).integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(src_np).pin_memory()
    dst = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    td, cd = torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda()
    so = torch.from_numpy(order).cuda() if order is not None else None
    P.paged_attention_decode_step(out, q, nk, nv, kd, vd, td, cd, mx, s.scale, dst, src, part, ws,
                                  seq_order=so)
    torch.cuda.synchronize()
    return (from_dev(out, s.dtype), from_dev(kd, s.dtype), from_dev(vd, s.dtype),
            dst.cpu().numpy(), src_np)


@pytest.mark.parametrize("name", ["llama13b", "gqa_prefix", "long_splitk", "f32_g2_d128"])
@pytest.mark.parametrize("part", [0, P.PARTITION_AUTO])
def test_decode_step_uploads_the_next_arrays_in_the_same_launch(name, part, decode_path):
    """The decode step with the next step's upload: output and caches
    bit-identical to the fused-write call (the same kernels and work), the
    uploaded bytes exact, for uploads larger than one grid row's threads."""
    s = CASES[name]
    wl, slots, tables, ctx, kc, vc = _setup(s)
    ko, vo = OC.reshape_and_cache(wl.new_k, wl.new_v, kc, vc, slots)
    ref = OA.paged_decode(wl.q, ko, vo, tables, ctx, s.scale, s.dtype)
    order = P.longest_first_order(ctx)
    paths = [P.PATH_AUTO] if s.dtype == "f32" else [P.PATH_VALU, P.PATH_MFMA]
    for path in paths:
        decode_path(path)
        for nbytes in (16, 16 * 40963):  # one piece; more than four per thread of the row
            log(f"decode step {name} partition={part} path={path} upload={nbytes} B")
            got, kd, vd, dst, src = _run_step(s, wl, tables, ctx, kc, vc, part, nbytes,
                                              seed=nbytes, order=order)
            assert np.array_equal(dst, src), "the next step's arrays"
            assert np.array_equal(_bits(kd), _bits(ko)) and np.array_equal(_bits(vd), _bits(vo))
            fused, _, _ = _run(s, wl, tables, ctx, kc, vc, part, True, order=order)
            assert np.array_equal(_bits(got), _bits(fused)), "decode step vs fused write"
            assert_close(OA.widen(got, s.dtype), ref, s.dtype, f"step {name} p{part} path{path}")


@pytest.mark.parametrize("name", ["tiny_fp32", "llama7b", "gqa_prefix", "long_splitk",
                                  "groups_g8_d64"])
@pytest.mark.parametrize("part", [0, P.PARTITION_AUTO])
def test_decode_step_without_new_tokens_uploads_and_decodes(name, part, decode_path):
    """A step whose caches already hold every token: the decode step with no
    new rows leaves the caches as they are, uploads the next arrays exactly,
    and gives the output of paged_attention_decode bit for bit."""
    s = CASES[name]
    wl, slots, tables, ctx, kc, vc = _setup(s)
    ko, vo = OC.reshape_and_cache(wl.new_k, wl.new_v, kc, vc, slots)
    ref = OA.paged_decode(wl.q, ko, vo, tables, ctx, s.scale, s.dtype)
    order = P.longest_first_order(ctx)
    paths = [P.PATH_AUTO] if s.dtype == "f32" else [P.PATH_VALU, P.PATH_MFMA]
    for path in paths:
        decode_path(path)
        for nbytes in (16, 16 * 40963):
            log(f"decode step without new tokens {name} partition={part} path={path} "
                f"upload={nbytes} B")
            got, kd, vd, dst, src = _run_step(s, wl, tables, ctx, ko, vo, part, nbytes,
                                              seed=nbytes + 1, order=order, rows=False)
            assert np.array_equal(dst, src), "the next step's arrays"
            assert np.array_equal(_bits(kd), _bits(ko)) and np.array_equal(_bits(vd), _bits(vo))
            # the plain decode over the same caches (re-writing the rows they hold)
            plain, _, _ = _run(s, wl, tables, ctx, ko, vo, part, False, order=order)
            assert np.array_equal(_bits(got), _bits(plain)), "decode step vs plain decode"
            assert_close(OA.widen(got, s.dtype), ref, s.dtype, f"step {name} p{part} path{path}")


def test_decode_step_refuses_pageable_memory_before_launch():
    s = CASES["llama13b"]
    wl, slots, tables, ctx, kc, vc = _setup(s)
    kd, vd = to_dev(kc, s.dtype), to_dev(vc, s.dtype)
    q = to_dev(wl.q, s.dtype)
    out = torch.full_like(q, 5.0)
    dst = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(P.PkvError, match="INVALID_ARG"):
        P.paged_attention_decode_step(out, q, to_dev(wl.new_k, s.dtype), to_dev(wl.new_v, s.dtype),
                                      kd, vd, torch.from_numpy(tables).cuda(),
                                      torch.from_numpy(ctx).cuda(), int(ctx.max()), s.scale, dst,
                                      torch.zeros(64, dtype=torch.uint8), 0)
    torch.cuda.synchronize()
    assert (out.float() == 5.0).all()
    assert np.array_equal(from_dev(kd, s.dtype), kc)
