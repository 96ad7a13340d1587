"""Helpers for the GPU parity tests: build one decode step on the device with
the product library and the same step on the CPU with the oracle.

Inputs come from ``workloads``.  The product side replays the workload with
the C++ allocator and the HIP kernels; the oracle side replays it with the
Python allocator model and the fp64 oracle.  Block tables and slots of the
two sides are asserted equal before any attention value is compared, and no
oracle input is taken from the product side.
"""
from __future__ import annotations

import dataclasses
import sys
from typing import Optional

import numpy as np
import torch

import oracle.allocator as OAL
import oracle.attention as OA
import oracle.cache_write as OC
import workloads as W


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint16).view(np.int16)).cuda().view(
        torch.bfloat16)


def from_dev(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Stored elements of a device tensor, back on the host (f32, or bf16 bits)."""
    if dtype == "f32":
        return t.detach().float().cpu().numpy()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@dataclasses.dataclass
class Step:
    shape: W.DecodeShape
    wl: W.Workload
    tables: np.ndarray        # oracle tables (equal to the product's)
    ctx: np.ndarray
    slots: Optional[np.ndarray]
    k_host: np.ndarray        # oracle view of the caches after the step's write
    v_host: np.ndarray
    q_host: np.ndarray
    # device side
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    tables_dev: torch.Tensor
    ctx_dev: torch.Tensor
    max_ctx: int


def poison_unused_tail(cache: np.ndarray, tables: np.ndarray, ctx: np.ndarray, dtype: str) -> None:
    """NaN in every slot past a sequence's context inside its last block."""
    bs = cache.shape[1]
    nan = np.float32(np.nan) if dtype == "f32" else W.BF16_NAN_BITS
    for b, c in enumerate(ctx):
        c = int(c)
        if c % bs:
            cache[tables[b, (c - 1) // bs], c % bs:] = nan


def build_step(shape: W.DecodeShape, poison: bool = True, pad: int = -1,
               q_scale: float = 1.0) -> Step:
    """Replay ``shape`` on both sides and run the product's cache write."""
    import paged_kv_cache_292_amd as P

    s = shape
    wl = W.make_workload(s)
    B = s.num_seqs
    oa = OAL.BlockAllocator(wl.num_blocks, s.block_size, wl.free_order)
    oa.replay(wl.ops)
    pa = P.Allocator(wl.num_blocks, s.block_size, wl.free_order)
    pa.replay(wl.ops)
    slots_o = slots_p = None
    if s.new_tokens:
        slots_o = np.array([oa.append(b, 1)[0] for b in range(B)], dtype=np.int64)
        slots_p = pa.append_tokens(list(range(B)), [1] * B)
        assert np.array_equal(slots_o, slots_p), "slot mapping differs from the oracle's"
    maxb = max(len(oa.tables[b]) for b in range(B)) + 2
    tables_o, ctx_o = oa.build_block_tables(list(range(B)), maxb, pad=pad)
    tables_p, ctx_p = pa.build_block_tables(list(range(B)), maxb, pad=pad)
    assert np.array_equal(tables_o, tables_p), "block tables differ from the oracle's"
    assert np.array_equal(ctx_o, ctx_p)
    pa.close()

    kc, vc = wl.k_cache, wl.v_cache
    if poison:
        poison_unused_tail(kc, tables_o, ctx_o, s.dtype)
        poison_unused_tail(vc, tables_o, ctx_o, s.dtype)
        if s.new_tokens:  # the new tokens' slots hold garbage until written
            nan = np.float32(np.nan) if s.dtype == "f32" else W.BF16_NAN_BITS
            for sl in slots_o:
                kc[sl // s.block_size, sl % s.block_size] = nan
                vc[sl // s.block_size, sl % s.block_size] = nan
    q_host = wl.q
    if q_scale != 1.0:
        q_host = (W.f32_to_bf16_bits(OA.widen(q_host, s.dtype).astype(np.float32) * q_scale)
                  if s.dtype == "bf16" else (q_host * q_scale).astype(np.float32))

    q = to_dev(q_host, s.dtype)
    k_dev = to_dev(kc, s.dtype)
    v_dev = to_dev(vc, s.dtype)
    if s.new_tokens:
        nk = to_dev(wl.new_k, s.dtype)
        nv = to_dev(wl.new_v, s.dtype)
        P.kv_reshape_and_cache(nk, nv, k_dev, v_dev, torch.from_numpy(slots_p).cuda())
        kc, vc = OC.reshape_and_cache(wl.new_k, wl.new_v, kc, vc, slots_o)
    torch.cuda.synchronize()
    return Step(s, wl, tables_o, ctx_o, slots_o, kc, vc, q_host, q, k_dev, v_dev,
                torch.from_numpy(tables_p).cuda(), torch.from_numpy(ctx_p).cuda(),
                int(ctx_o.max()))


def run_decode(st: Step, partition_size: int, order=None) -> np.ndarray:
    """Product decode of the step (``order``: optional launch order, host
    int32); returns the output as float64."""
    import paged_kv_cache_292_amd as P

    s = st.shape
    out = torch.empty_like(st.q)
    ws_bytes = P.decode_workspace_bytes(s.num_seqs, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                        s.block_size, st.max_ctx, partition_size,
                                        P.F32 if s.dtype == "f32" else P.BF16)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes else None
    so = torch.from_numpy(np.ascontiguousarray(order, dtype=np.int32)).cuda() if order is not None else None
    P.paged_attention_decode(out, st.q, st.k_cache, st.v_cache, st.tables_dev, st.ctx_dev,
                             st.max_ctx, s.scale, partition_size, ws, seq_order=so)
    torch.cuda.synchronize()
    return OA.widen(from_dev(out, s.dtype), s.dtype)


def oracle_rows(st: Step, pairs) -> np.ndarray:
    """Oracle outputs for the given (sequence, query head) pairs, float64."""
    s = st.shape
    G = s.group
    res = np.zeros((len(pairs), s.head_dim))
    cache_b = {}
    for i, (b, h) in enumerate(pairs):
        if b not in cache_b:
            c = int(st.ctx[b])
            k = OA.widen(OA.gather_sequence(st.k_host, st.tables[b], c, s.block_size), s.dtype)
            v = OA.widen(OA.gather_sequence(st.v_host, st.tables[b], c, s.block_size), s.dtype)
            cache_b = {b: (k, v)}
        k, v = cache_b[b]
        qv = OA.widen(st.q_host[b, h], s.dtype)
        res[i] = OA.attend(qv, k[:, h // G, :], v[:, h // G, :], s.scale) if len(k) else 0.0
    return res


def oracle_full(st: Step) -> np.ndarray:
    s = st.shape
    return OA.paged_decode(st.q_host, st.k_host, st.v_host, st.tables, st.ctx, s.scale, s.dtype)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> None:
    """fp32: per (sequence, head) row, max |err| <= 1e-5 * max |ref|.
    bf16: max |err| <= 2e-2 over all elements, and per row a normwise relative
    error <= 1e-2 (stricter self-check; bf16 output rounding alone is 2^-9)."""
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rows_err = err.reshape(-1, got.shape[-1]).max(axis=1)
    rows_ref = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1)
    if dtype == "f32":
        bad = rows_err > 1e-5 * rows_ref + 1e-30
        assert not bad.any(), (f"{what}: {bad.sum()} rows over 1e-5 relative; worst "
                               f"{(rows_err / np.maximum(rows_ref, 1e-30)).max():.3e}")
    else:
        assert err.max() <= 2e-2, f"{what}: max abs error {err.max():.3e} > 2e-2"
        nerr = np.linalg.norm((got - ref).reshape(-1, got.shape[-1]), axis=1)
        nref = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
        rel = nerr / np.maximum(nref, 1e-30)
        assert rel.max() <= 1e-2, f"{what}: normwise relative error {rel.max():.3e} > 1e-2"
    log(f"  {what}: max abs err {err.max():.3e}, max |ref| {np.abs(ref).max():.3e}")
