"""GPU parity of the shared-prefix decode: sequences whose tables start
with the same blocks get their prefix partition computed once per tile of
members (16 / G per tile), the rest as in the partitioned decode, merged by
log-sum-exp.  The prefix is partition 0; later partitions are max(2048,
prefix) tokens.  Every case is checked against the fp64 oracle (which knows
nothing of the sharing) and against the ordinary partitioned decode with
prefix-length partitions (equal up to rounding)."""
import numpy as np
import pytest

import workloads as W
from gpu_cases import assert_close, build_step, log, oracle_full, oracle_rows, run_decode

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)
import paged_kv_cache_292_amd as P  # noqa: E402  (fails loudly when the library is missing)


@pytest.fixture
def decode_path():
    """Select a decode kernel for one test, restore the automatic choice after."""
    yield P.set_decode_path
    P.set_decode_path(P.PATH_AUTO)


def run_shared(st, members, prefix, order=None, upload=None):
    """The shared-prefix call; upload = (device dst, pinned src) runs the
    step form that also copies src into dst within the launch."""
    s = st.shape
    out = torch.empty_like(st.q)
    ws_bytes = P.decode_workspace_bytes(s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                        s.block_size, st.max_ctx, prefix, P.BF16)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    flag = np.zeros(s.num_seqs, dtype=np.int32)
    flag[np.asarray(members, dtype=np.int64)] = 1
    m_dev = torch.from_numpy(np.ascontiguousarray(members, dtype=np.int32)).cuda()
    f_dev = torch.from_numpy(flag).cuda()
    so = torch.from_numpy(np.ascontiguousarray(order, dtype=np.int32)).cuda() if order is not None else None
    if upload is None:
        P.paged_attention_decode_shared_prefix(out, st.q, st.k_cache, st.v_cache, st.tables_dev,
                                               st.ctx_dev, st.max_ctx, s.scale, m_dev, f_dev,
                                               prefix, ws, seq_order=so)
    else:
        P.paged_attention_decode_shared_prefix_step(out, st.q, st.k_cache, st.v_cache,
                                                    st.tables_dev, st.ctx_dev, st.max_ctx,
                                                    s.scale, m_dev, f_dev, prefix, upload[0],
                                                    upload[1], ws, seq_order=so)
    torch.cuda.synchronize()
    from gpu_cases import OA, from_dev
    return OA.widen(from_dev(out, s.dtype), s.dtype)


def shape_with_sharing(B, hq, hkv, D, bs, prefix, sharers, lo, hi, seed):
    return W.DecodeShape("shared", "bf16", B, hq, hkv, D, bs, "uniform", ctx_lo=lo, ctx_hi=hi,
                         shared_prefix_tokens=prefix, num_sharers=sharers, seed=seed)


@pytest.mark.parametrize("B,hq,hkv,D,bs,prefix,sharers", [
    (16, 32, 8, 128, 32, 1024, 6),    # the GQA shape's structure, scaled
    (12, 16, 2, 128, 16, 512, 9),     # G = 8: two members per tile, an odd count
    (10, 32, 2, 128, 32, 256, 7),     # G = 16: one member per tile
    (9, 6, 2, 64, 16, 96, 8),         # G = 3: five members per tile, head_dim 64
    (8, 8, 4, 128, 16, 16, 8),        # G = 2 (matrix cores forced), one-block prefix, all share
])
def test_shared_prefix_matches_oracle(B, hq, hkv, D, bs, prefix, sharers, decode_path):
    if hq // hkv < 4:
        decode_path(P.PATH_MFMA)  # the automatic choice takes the vector kernel there
    s = shape_with_sharing(B, hq, hkv, D, bs, prefix, sharers, prefix + 1, prefix + 900,
                           seed=hq * 31 + prefix)
    log(f"shared prefix B={B} G={hq // hkv} D={D} bs={bs} prefix={prefix} sharers={sharers}")
    st = build_step(s, poison=True, pad=-5)
    members = st.wl.sharers
    ref = oracle_full(st)
    got = run_shared(st, members, prefix)
    assert_close(got, ref, "bf16", f"shared prefix G{hq // hkv} p{prefix}")
    base = run_decode(st, prefix)
    assert_close(got, base.astype(np.float64), "bf16", "shared prefix vs partitioned decode")
    order = P.longest_first_order(st.ctx)
    assert_close(run_shared(st, members, prefix, order), ref, "bf16", "shared prefix, ordered")


@pytest.mark.parametrize("prefix,lo,hi,bs", [
    (256, 2500, 7000, 16),    # later partitions of 2048 tokens, up to four of them
    (2560, 2561, 9000, 32),   # prefix over 2048: later partitions of the prefix's length
])
def test_shared_prefix_with_several_later_partitions(prefix, lo, hi, bs):
    """Contexts that run several partitions past the prefix: the partition
    boundaries after the prefix partition fall every max(2048, prefix) tokens
    from its end, and every partition's partials meet in the merge."""
    s = shape_with_sharing(6, 32, 8, 128, bs, prefix, 4, lo, hi, seed=prefix + lo)
    log(f"shared prefix, later partitions: prefix={prefix} contexts {lo}..{hi} bs={bs}")
    st = build_step(s, poison=True, pad=-3)
    members = st.wl.sharers
    ref = oracle_full(st)
    got = run_shared(st, members, prefix, P.longest_first_order(st.ctx))
    assert_close(got, ref, "bf16", f"shared prefix {prefix}, long contexts")
    assert_close(run_shared(st, members, prefix), ref, "bf16", "unordered")


def test_shared_prefix_with_no_members_is_the_partitioned_decode():
    s = shape_with_sharing(6, 32, 8, 128, 32, 1024, 0, 200, 3000, seed=7)
    st = build_step(s, poison=True)
    got = run_shared(st, np.zeros(0, dtype=np.int64), 512)
    np.testing.assert_array_equal(got, run_decode(st, 512))


def test_shared_prefix_full_gqa_shape_sampled():
    """The GQA decode batch at full size (256 sequences, 128 sharing a
    1,024-token prefix): sampled rows of members and non-members."""
    s = W.shape(3)
    st = build_step(s, poison=True, pad=-1)
    members = st.wl.sharers
    got = run_shared(st, members, s.shared_prefix_tokens, P.longest_first_order(st.ctx))
    assert np.isfinite(got).all()
    rng = np.random.default_rng(3)
    others = np.setdiff1d(np.arange(s.num_seqs), members)
    bs_ = list(members[:4]) + list(rng.choice(members, 4)) + list(rng.choice(others, 4))
    pairs = [(int(b), h) for b in bs_ for h in (0, 13, s.num_q_heads - 1)]
    assert_close(np.stack([got[b, h] for b, h in pairs]), oracle_rows(st, pairs), "bf16",
                 "full GQA shared prefix")


@pytest.mark.parametrize("B,hq,hkv,D,bs,prefix,sharers", [
    (16, 32, 8, 128, 32, 1024, 6),
    (12, 16, 2, 128, 16, 512, 9),
    (9, 6, 2, 64, 16, 96, 8),
])
def test_shared_prefix_step_uploads_the_next_arrays_in_the_same_launch(B, hq, hkv, D, bs, prefix,
                                                                      sharers, decode_path):
    """The step form: output bit-identical to the shared-prefix call (the
    same workgroups, shifted one grid row), the uploaded bytes exact, for an
    upload of one piece and one larger than a grid row's threads."""
    if hq // hkv < 4:
        decode_path(P.PATH_MFMA)
    s = shape_with_sharing(B, hq, hkv, D, bs, prefix, sharers, prefix + 1, prefix + 900,
                           seed=hq * 37 + prefix)
    st = build_step(s, poison=True, pad=-5)
    members = st.wl.sharers
    ref = oracle_full(st)
    order = P.longest_first_order(st.ctx)
    plain = run_shared(st, members, prefix, order)
    for nbytes in (16, 16 * 40963):
        log(f"shared prefix step G={hq // hkv} prefix={prefix} upload={nbytes} B")
        src_np = np.random.default_rng(nbytes).integers(0, 256, nbytes, dtype=np.uint8)
        src = torch.from_numpy(src_np).pin_memory()
        dst = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
        got = run_shared(st, members, prefix, order, upload=(dst, src))
        assert np.array_equal(dst.cpu().numpy(), src_np), "the next step's arrays"
        np.testing.assert_array_equal(got, plain)
        assert_close(got, ref, "bf16", f"shared prefix step G{hq // hkv}")
