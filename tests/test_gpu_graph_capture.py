"""The decode calls under HIP graph capture (torch.cuda.CUDAGraph), the use
the no-allocation entry point is for: each call is captured once after an
eager warm-up, then the graph is replayed several times with eager work
(output poisoning, other decode calls over the same static scratch, a new
upload source) and synchronizations between the replays; every replay must
give the eager result bit for bit and, for the decode step, upload the
source's contents at replay time."""
import numpy as np
import pytest

import workloads as W
from gpu_cases import OA, assert_close, build_step, from_dev, log, oracle_full

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)
import paged_kv_cache_292_amd as P  # noqa: E402  (fails loudly when the library is missing)


def _capture(call):
    """Warm up on a side stream (default priority), then capture ``call``."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    return g


def _bits(t):
    return t.view(torch.int16).cpu().numpy().copy()


def test_noalloc_decode_replays_under_graph_capture():
    s = W.scaled(W.shape(4), num_seqs=4)  # G = 8, 512-token partitions: scratch and merge
    other = W.scaled(W.shape(3), num_seqs=5, num_sharers=2)
    st = build_step(s, poison=True, pad=-1)
    st2 = build_step(other, poison=True, pad=-1)
    order = torch.from_numpy(P.longest_first_order(st.ctx)).cuda()
    out = torch.empty_like(st.q)

    def call():
        P.paged_attention_decode_noalloc(out, st.q, st.k_cache, st.v_cache, st.tables_dev,
                                         st.ctx_dev, st.max_ctx, s.scale, 512, seq_order=order)

    call()
    torch.cuda.synchronize()
    eager = _bits(out)
    assert_close(OA.widen(from_dev(out, s.dtype), s.dtype), oracle_full(st), s.dtype,
                 "noalloc eager")
    g = _capture(call)
    out2 = torch.empty_like(st2.q)
    for i in range(3):
        log(f"noalloc graph replay {i}")
        out.fill_(float("nan"))
        # another call over the same static scratch between the replays
        P.paged_attention_decode_noalloc(out2, st2.q, st2.k_cache, st2.v_cache, st2.tables_dev,
                                         st2.ctx_dev, st2.max_ctx, other.scale, 512)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), eager), f"replay {i}"


@pytest.mark.parametrize("rows", [False, True])
def test_decode_step_replays_under_graph_capture(rows):
    """The decode step with its upload (and, with rows, its cache write of
    the step's new tokens, which rewrites the same slots on every replay)."""
    base = W.scaled(W.shape(2), num_seqs=12)
    s = base if rows else W.scaled(W.shape(1), num_seqs=6)
    st = build_step(s, poison=True, pad=-1)
    order = torch.from_numpy(P.longest_first_order(st.ctx)).cuda()
    nbytes = 16 * 5003
    src = torch.zeros(nbytes, dtype=torch.uint8).pin_memory()
    dst = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(st.q)
    ws_bytes = P.decode_workspace_bytes(s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                        s.block_size, st.max_ctx, P.PARTITION_AUTO, P.BF16)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    nk = nv = None
    if rows:  # the step's new rows rewritten into the slots the cache write filled
        from gpu_cases import to_dev
        nk, nv = to_dev(st.wl.new_k, s.dtype), to_dev(st.wl.new_v, s.dtype)

    def call():
        P.paged_attention_decode_step(out, st.q, nk, nv, st.k_cache, st.v_cache, st.tables_dev,
                                      st.ctx_dev, st.max_ctx, s.scale, dst, src,
                                      P.PARTITION_AUTO, ws, seq_order=order)

    call()
    torch.cuda.synchronize()
    eager = _bits(out)
    k_before = _bits(st.k_cache)
    g = _capture(call)
    rng = np.random.default_rng(17)
    for i in range(3):
        log(f"decode step graph replay {i} rows={rows}")
        fresh = rng.integers(0, 256, nbytes, dtype=np.uint8)
        src.numpy()[:] = fresh  # the next step's arrays, written after capture
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), eager), f"replay {i}"
        assert np.array_equal(dst.cpu().numpy(), fresh), f"upload at replay {i}"
        assert np.array_equal(_bits(st.k_cache), k_before), "cache after the rewrite"
