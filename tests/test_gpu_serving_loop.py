"""Several decode steps of a serving loop, the way the benchmark runs them:
the host allocator prepares each step's slots, tables, lengths and
longest-first order one step ahead into pinned memory, and each decode-step
launch writes the step's new tokens, decodes, and uploads the next step's
arrays for the following launch ("vLLM in Production …", section
"Continuous Batching Keeps the GPU Full": the batch is re-formed at every
step; section "PagedAttention — Virtual Memory for the KV Cache": tokens go
into blocks as they arrive).  Every step's output is checked against the
fp64 oracle over the oracle allocator's tables and the oracle's cache write;
the caches must match bit for bit at the end.  Unlike the full-size tests
(the first step only) this checks that each launch decodes from the arrays
the previous launch uploaded."""
import numpy as np
import pytest

import oracle.allocator as OAL
import oracle.attention as OA
import oracle.cache_write as OC
import workloads as W
from gpu_cases import assert_close, from_dev, log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)
import paged_kv_cache_292_amd as P  # noqa: E402  (fails loudly when the library is missing)

STEPS = 6

SHAPES = {
    # the 13B batch's structure (G = 1, vector kernel, single pass)
    "g1": W.scaled(W.shape(2), num_seqs=10),
    # grouped heads with contexts past 2048 tokens (matrix cores, partitions and merge)
    "g4": W.DecodeShape("loop_g4", "bf16", 6, 16, 4, 128, 32, "uniform", ctx_lo=300,
                        ctx_hi=5000, new_tokens=True, seed=71),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_serving_loop_steps_match_the_oracle(name):
    s = SHAPES[name]
    wl = W.make_workload(s, extra_tokens=STEPS + 1)
    B, bs = s.num_seqs, s.block_size
    oa = OAL.BlockAllocator(wl.num_blocks, bs, wl.free_order)
    oa.replay(wl.ops)
    pa = P.Allocator(wl.num_blocks, bs, wl.free_order)
    pa.replay(wl.ops)
    seqs = np.arange(B, dtype=np.int64)
    mb = int(((wl.ctx + STEPS + bs - 1) // bs).max())

    # staging layout: slots int64 [B] | tables int32 [B, mb] | lengths int32 [B] | order int32 [B]
    o_tb = 8 * B
    o_cx = o_tb + 4 * B * mb
    o_or = o_cx + 4 * B
    nbytes = (o_or + 4 * B + 15) // 16 * 16
    pinned = [torch.zeros(nbytes, dtype=torch.uint8).pin_memory() for _ in range(2)]
    stage = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]

    def views(t):
        return (t[o_tb:o_cx].view(torch.int32).view(B, mb), t[o_cx:o_or].view(torch.int32),
                t[o_or:o_or + 4 * B].view(torch.int32))

    prepared = {}

    def prepare(k):
        """Step k's arrays into pinned buffer k % 2, checked against the oracle allocator."""
        host = np.zeros(nbytes, dtype=np.uint8)
        slots = host[:o_tb].view(np.int64)
        tables = host[o_tb:o_cx].view(np.int32).reshape(B, mb)
        ctx = host[o_cx:o_or].view(np.int32)
        order = host[o_or:o_or + 4 * B].view(np.int32)
        mx = pa.decode_step_prepare(seqs, mb, slots, tables, ctx, order_out=order)
        so = np.array([oa.append(b, 1)[0] for b in range(B)], dtype=np.int64)
        to, co = oa.build_block_tables(list(range(B)), mb, pad=-1)
        assert np.array_equal(slots, so) and np.array_equal(tables, to) and np.array_equal(ctx, co)
        pinned[k % 2].numpy()[:] = host
        prepared[k] = (mx, so, to, co)

    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    kd, vd = to_dev(kc, s.dtype), to_dev(vc, s.dtype)
    q = to_dev(wl.q, s.dtype)
    out = torch.empty_like(q)
    max_final = int((wl.ctx + STEPS).max())
    wsb = P.decode_workspace_bytes(B, s.num_q_heads, s.num_kv_heads, s.head_dim, bs, max_final,
                                   P.PARTITION_AUTO, P.BF16)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")

    prepare(0)
    P.upload_pinned(stage[0], pinned[0])
    for i in range(STEPS):
        nk, nv = (wl.new_k, wl.new_v) if i == 0 else W.step_tokens(s, i)
        prepare(i + 1)  # the host runs one step ahead
        mx, slots, tables, ctx = prepared.pop(i)
        tb, cx, od = views(stage[i % 2])
        log(f"serving loop {name} step {i}: max context {mx}")
        P.paged_attention_decode_step(out, q, to_dev(nk, s.dtype), to_dev(nv, s.dtype), kd, vd, tb,
                                      cx, mx, s.scale, stage[(i + 1) % 2], pinned[(i + 1) % 2],
                                      P.PARTITION_AUTO, ws, seq_order=od)
        torch.cuda.synchronize()
        assert np.array_equal(stage[(i + 1) % 2].cpu().numpy(), pinned[(i + 1) % 2].numpy())
        kc, vc = OC.reshape_and_cache(nk, nv, kc, vc, slots)
        ref = OA.paged_decode(wl.q, kc, vc, tables, ctx, s.scale, s.dtype)
        assert_close(OA.widen(from_dev(out, s.dtype), s.dtype), ref, s.dtype,
                     f"{name} step {i}")
    assert np.array_equal(from_dev(kd, s.dtype), kc) and np.array_equal(from_dev(vd, s.dtype), vc)
    pa.close()
