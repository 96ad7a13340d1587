"""PagedAttention decode for AMD MI355X (gfx950): Python binding of libpkv.

Thin ctypes marshalling over the C ABI declared in ``include/pkv.h``; every
step of the hot path runs in the library's HIP kernels or its C++ allocator.
Device arguments are torch tensors (their ``data_ptr()``), launched on the
current torch stream unless a stream is given.  The library must be built
first (``python paged_kv_cache_292_amd/build.py``); importing this package
without it raises ``ImportError`` — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "LIB_PATH", "lib", "PkvError", "F32", "BF16", "PARTITION_AUTO",
    "kv_reshape_and_cache", "paged_attention_decode", "paged_attention_decode_write",
    "paged_attention_decode_shared_prefix",
    "decode_workspace_bytes",
    "decode_partition_size", "stream_read", "copy_blocks", "set_decode_path", "get_decode_path", "upload_pinned", "longest_first_order",
    "paged_attention_prefill", "prefill_workspace_bytes", "prefill_partition_size",
    "swap_blocks", "SWAP_OUT", "SWAP_IN",
    "PATH_AUTO", "PATH_VALU", "PATH_MFMA", "Allocator", "EXPORTS", "version",
    "blocks_for_budget", "validate_decode_inputs", "paged_attention_decode_noalloc",
    "NOALLOC_SCRATCH_BYTES", "paged_attention_decode_step",
    "paged_attention_decode_shared_prefix_step",
]

LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

F32 = 0
BF16 = 1
PARTITION_AUTO = -1
NOALLOC_SCRATCH_BYTES = 64 << 20  # PKV_NOALLOC_SCRATCH_BYTES
PATH_AUTO, PATH_VALU, PATH_MFMA = 0, 1, 2

STATUS = {
    0: "OK", -1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "OUT_OF_BLOCKS", -4: "NOT_FOUND",
    -5: "SHARED_WRITE", -6: "WORKSPACE", -7: "HIP", -8: "SWAPPED",
}
SWAP_OUT, SWAP_IN = 0, 1

# name -> (restype, argtypes), the exported C ABI
_i32, _i64, _sz, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p
_P = ctypes.POINTER
EXPORTS = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_kv_reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                        _i64, _i64, _i32, _vp]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_partition_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_stream_read": (_i32, [_vp, _sz, _vp, _i32, _vp]),
    "pkv_paged_attention_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                          _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz,
                                          _i32, _vp]),
    "pkv_paged_attention_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32,
                                                  _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                                  _i32, _vp]),
    "pkv_paged_attention_decode_shared_prefix": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                                                        _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                        _f32, _vp, _vp, _i32, _i32, _vp, _sz,
                                                        _i32, _vp]),
    "pkv_paged_attention_decode_shared_prefix_step": (
        _i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
               _f32, _vp, _vp, _i32, _i32, _vp, _sz, _vp, _vp, _sz, _i32, _vp]),
    "pkv_paged_attention_decode_write": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp,
                                                _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                                _i32, _i32, _f32, _i32, _vp, _sz, _i32, _vp]),
    "pkv_paged_attention_decode_step": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp,
                                               _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                               _i32, _i32, _f32, _i32, _vp, _sz, _vp, _vp, _sz,
                                               _i32, _vp]),
    "pkv_longest_first_order": (_i32, [_P(_i32), _i32, _P(_i32)]),
    "pkv_prefill_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_prefill_partition_size": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attention_prefill": (_i32, [_vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _i32, _vp,
                                           _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                           _i32, _vp, _sz, _i32, _vp]),
    "pkv_set_decode_path": (_i32, [_i32]),
    "pkv_get_decode_path": (_i32, []),
    "pkv_upload_pinned": (_i32, [_vp, _vp, _sz, _vp]),
    "pkv_copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pkv_swap_blocks": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                               _i32, _vp]),
    "pkv_allocator_set_host_pool": (_i32, [_vp, _i32, _P(_i32)]),
    "pkv_swap_out": (_i32, [_vp, _P(_i64), _i32, _P(_i64), _i32, _P(_i32)]),
    "pkv_swap_in": (_i32, [_vp, _P(_i64), _i32, _P(_i64), _i32, _P(_i32)]),
    "pkv_seq_is_swapped": (_i32, [_vp, _i64]),
    "pkv_allocator_enable_prefix_cache": (_i32, [_vp]),
    "pkv_seq_add_prompt": (_i32, [_vp, _i64, _P(_i32), _i32, _P(_i64), _P(_i32)]),
    "pkv_prefix_cache_stats": (_i32, [_vp, _P(_i64), _P(_i64), _P(_i32)]),
    "pkv_num_free_host_blocks": (_i32, [_vp]),
    "pkv_host_block_refcount": (_i32, [_vp, _i32]),
    "pkv_allocator_create": (_i32, [_i32, _i32, _P(_i32), _P(_vp)]),
    "pkv_allocator_destroy": (None, [_vp]),
    "pkv_seq_add": (_i32, [_vp, _i64]),
    "pkv_seq_fork_prefix": (_i32, [_vp, _i64, _i64, _i32]),
    "pkv_seq_append": (_i32, [_vp, _i64, _i32, _P(_i64)]),
    "pkv_append_tokens": (_i32, [_vp, _P(_i64), _P(_i32), _i32, _P(_i64)]),
    "pkv_append_tokens_cow": (_i32, [_vp, _P(_i64), _P(_i32), _i32, _P(_i64), _P(_i64), _i32,
                                     _P(_i32)]),
    "pkv_seq_free": (_i32, [_vp, _i64]),
    "pkv_build_block_tables": (_i32, [_vp, _P(_i64), _i32, _i32, _i32, _P(_i32), _P(_i32)]),
    "pkv_decode_step_prepare": (_i32, [_vp, _P(_i64), _i32, _i32, _i32, _P(_i64), _P(_i32),
                                       _P(_i32), _P(_i32), _P(_i32)]),
    "pkv_num_free_blocks": (_i32, [_vp]),
    "pkv_block_refcount": (_i32, [_vp, _i32]),
    "pkv_seq_context_len": (_i64, [_vp, _i64]),
    "pkv_seq_num_blocks": (_i32, [_vp, _i64]),
    "pkv_shared_prefix_members": (_i32, [_vp, _P(_i64), _i32, _i32, _P(_i32), _P(_i32), _P(_i32)]),
    "pkv_blocks_for_budget": (_i32, [_sz, _i32, _i32, _i32, _i32, _i32]),
    "pkv_validate_decode_inputs": (_i32, [_P(_i32), _i32, _i32, _P(_i32), _P(_i32), _i32, _i32,
                                          _i32, _P(_i32), _P(_i32), _i32, _i32]),
}


def _load():
    # torch brings its own HIP runtime; loading it first makes libpkv bind to
    # that same runtime (matched by soname) instead of a second copy.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python paged_kv_cache_292_amd/build.py`")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.code = STATUS.get(status, str(status))
        msg = lib.pkv_last_error().decode(errors="replace")
        super().__init__(f"{where}: {self.code}: {msg}")


def _check(st: int, where: str) -> None:
    if st != 0:
        raise PkvError(st, where)


def version() -> str:
    return lib.pkv_version().decode()


# ------------------------------------------------------------------ device calls
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _index_ptr(t, n: int, what: str, where: str, rows: bool = False, wide: bool = False,
               cols: Optional[int] = None):
    """Device pointer of an index array the kernels read up to entry (or,
    for ``rows``, row) ``n - 1``: a contiguous int32 (``wide``: int64) device
    tensor, with ``cols`` columns when given.  A host tensor, another dtype
    or too few entries would reach the kernel as a bad address, so they are
    refused here.  ``None`` stays ``None``."""
    import torch
    if t is None:
        return None
    want = torch.int64 if wide else torch.int32
    have = (t.shape[0] if t.dim() == 2 else -1) if rows else t.numel()
    if (t.dtype != want or not t.is_cuda or not t.is_contiguous() or have < n
            or (cols is not None and (t.dim() != 2 or t.shape[1] != cols))):
        shape = f"[>= {n}, {cols}]" if cols is not None else f"at least {n} " + (
            "rows" if rows else "entries")
        raise ValueError(f"{where}: {what} must be a contiguous {str(want)[6:]} device tensor, "
                         f"{shape} (got {t.dtype}, {t.device}, shape {tuple(t.shape)})")
    return t.data_ptr()


def _dense_ptr(t, shape, dtype, what: str, where: str, rows: bool = False):
    """Device pointer of a dense operand the kernels read or write in full:
    a tensor of element type ``dtype`` (the cache's) and exactly ``shape``,
    contiguous (``rows``: only each row of the last two dimensions, as a
    strided batch of ``[Hkv, D]`` rows), on the device.  Another element type
    or shape would make a kernel read or write past the end of the buffer,
    and a host tensor would reach it as a bad address, so all are refused
    here.  Checked in that order, so each condition has its own message."""
    if t.dtype != dtype:
        raise ValueError(f"{where}: {what} must have the cache's element type {dtype} "
                         f"(got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{where}: {what} must have shape {list(shape)} (got {list(t.shape)})")
    if rows:
        dense = t.stride(-1) == 1 and (t.shape[-2] <= 1 or t.stride(-2) == t.shape[-1])
    else:
        dense = t.is_contiguous()
    if not dense:
        raise ValueError(f"{where}: {what} must be " + (
            "row-contiguous (stride(-1) == 1, stride(-2) == head_dim)" if rows else "contiguous"))
    if not t.is_cuda:
        raise ValueError(f"{where}: {what} must be a device tensor (got {t.device})")
    return t.data_ptr()


def _caches(k_cache, v_cache, where: str):
    """Shape ``(N, bs, Hkv, D)`` and element-type code of a K/V cache pair
    after checking both (same shape and type, contiguous, on the device)."""
    import torch
    if k_cache.dim() != 4 or k_cache.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"{where}: k_cache must be a float32 or bfloat16 [num_blocks, "
                         f"block_size, num_kv_heads, head_dim] tensor (got {k_cache.dtype}, "
                         f"{list(k_cache.shape)})")
    if v_cache.dtype != k_cache.dtype:
        raise ValueError(f"{where}: v_cache must have the cache's element type {k_cache.dtype} "
                         f"(got {v_cache.dtype})")
    if v_cache.shape != k_cache.shape:
        raise ValueError(f"{where}: v_cache must have shape {list(k_cache.shape)} "
                         f"(got {list(v_cache.shape)})")
    _dense_ptr(k_cache, k_cache.shape, k_cache.dtype, "k_cache", where)
    _dense_ptr(v_cache, k_cache.shape, k_cache.dtype, "v_cache", where)
    return tuple(k_cache.shape), _dtype_code(k_cache)


def _workspace(workspace, where: str):
    """(pointer, bytes) of an optional device workspace (``None``: none)."""
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError(f"{where}: workspace must be a contiguous device tensor "
                         f"(got {workspace.device})")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _decode_indices(block_tables, context_lens, seq_order, B: int, where: str):
    """Pointers of a decode call's tables, lengths and launch order."""
    return (_index_ptr(block_tables, B, "block_tables", where, rows=True),
            _index_ptr(context_lens, B, "context_lens", where),
            _index_ptr(seq_order, B, "seq_order", where))


def _q_out(q, out, shape, dtype, where: str):
    """Pointers of the queries and the output, both ``shape``, contiguous."""
    return (_dense_ptr(q, shape, dtype, "q", where), _dense_ptr(out, shape, dtype, "out", where))


def _stream_ptr(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def kv_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """Write ``key``/``value`` ``[T, Hkv, D]`` into the caches at ``slot_mapping`` (int64).
    Token rows may be strided; each token's ``[Hkv, D]`` must be contiguous."""
    fn = "kv_reshape_and_cache"
    T = key.shape[0]
    slots = _index_ptr(slot_mapping, T, "slot_mapping", fn, wide=True)
    (N, bs, Hkv, D), dt = _caches(k_cache, v_cache, fn)
    kp = _dense_ptr(key, (T, Hkv, D), k_cache.dtype, "key", fn, rows=True)
    vp = _dense_ptr(value, (T, Hkv, D), k_cache.dtype, "value", fn, rows=True)
    _check(lib.pkv_kv_reshape_and_cache(
        kp, vp, k_cache.data_ptr(), v_cache.data_ptr(), slots, T, Hkv, D, bs, N,
        key.stride(0) if T else Hkv * D, value.stride(0) if T else Hkv * D,
        dt, _stream_ptr(stream)), fn)


def longest_first_order(context_lens) -> np.ndarray:
    """Host: indices sorted by context length, longest first (ties by index)."""
    c = np.ascontiguousarray(context_lens, dtype=np.int32)
    out = np.empty(len(c), dtype=np.int32)
    _check(lib.pkv_longest_first_order(c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(c),
                                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
           "longest_first_order")
    return out


def decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_context_len, partition_size=PARTITION_AUTO, dtype=BF16) -> int:
    return int(lib.pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              block_size, max_context_len, partition_size,
                                              dtype))


def decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_context_len, partition_size=PARTITION_AUTO, dtype=BF16) -> int:
    return int(lib.pkv_decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             block_size, max_context_len, partition_size, dtype))


def stream_read(src, out, workgroups: int, stream=None) -> None:
    """Read every byte of the device tensor ``src`` once (16-byte
    non-temporal loads, nothing else): the streaming-read reference of the
    decode roofline.  ``out`` is a device uint32/int32 tensor of at least
    ``workgroups`` entries; entry w receives the XOR of the 32-bit words
    workgroup w read."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("stream_read: src must be a contiguous device tensor")
    if (not out.is_cuda or not out.is_contiguous() or out.element_size() != 4
            or out.numel() < workgroups):
        raise ValueError(f"stream_read: out must be a contiguous 32-bit device tensor of at "
                         f"least {workgroups} entries")
    _check(lib.pkv_stream_read(src.data_ptr(), src.numel() * src.element_size(), out.data_ptr(),
                               int(workgroups), _stream_ptr(stream)), "stream_read")


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens,
                           max_context_len: int, scale: float,
                           partition_size: int = PARTITION_AUTO, workspace=None,
                           stream=None, seq_order=None) -> None:
    """``out[b, h] = softmax(scale · K_b q[b, h]) V_b`` through the block tables.

    ``workspace`` is a device byte tensor of at least
    ``decode_workspace_bytes(...)`` bytes when partitions are used;
    ``seq_order`` an optional device int32 launch order (longest first is
    fastest, see ``longest_first_order``)."""
    fn = "paged_attention_decode"
    B, Hq = q.shape[0], q.shape[1]
    idx = _decode_indices(block_tables, context_lens, seq_order, B, fn)
    (N, bs, Hkv, D), dt = _caches(k_cache, v_cache, fn)
    qp, op = _q_out(q, out, (B, Hq, D), k_cache.dtype, fn)
    ws_ptr, ws_bytes = _workspace(workspace, fn)
    _check(lib.pkv_paged_attention_decode(
        op, qp, k_cache.data_ptr(), v_cache.data_ptr(), idx[0], block_tables.shape[1], idx[1],
        idx[2], int(max_context_len), B, Hq, Hkv, D, bs, N, float(scale), int(partition_size),
        ws_ptr, ws_bytes, dt, _stream_ptr(stream)), fn)


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens,
                                   max_context_len: int, scale: float,
                                   partition_size: int = PARTITION_AUTO, stream=None,
                                   seq_order=None) -> None:
    """``paged_attention_decode`` with no workspace argument: the library's
    static per-GPU scratch array (``NOALLOC_SCRATCH_BYTES``) holds the
    partials, so the call allocates nothing.  Calls that overlap on one GPU
    race on that array."""
    fn = "paged_attention_decode_noalloc"
    B, Hq = q.shape[0], q.shape[1]
    idx = _decode_indices(block_tables, context_lens, seq_order, B, fn)
    (N, bs, Hkv, D), dt = _caches(k_cache, v_cache, fn)
    qp, op = _q_out(q, out, (B, Hq, D), k_cache.dtype, fn)
    _check(lib.pkv_paged_attention_decode_noalloc(
        op, qp, k_cache.data_ptr(), v_cache.data_ptr(), idx[0], block_tables.shape[1], idx[1],
        idx[2], int(max_context_len), B, Hq, Hkv, D, bs, N, float(scale), int(partition_size),
        dt, _stream_ptr(stream)), fn)


def _next_upload(next_dst, next_src_pinned, fn):
    """Pointers and byte count of the next step's upload (a contiguous device
    tensor and a contiguous pinned host tensor of the same byte size)."""
    nbytes = next_src_pinned.numel() * next_src_pinned.element_size()
    if (next_dst.numel() * next_dst.element_size() != nbytes or not next_dst.is_cuda
            or not next_dst.is_contiguous() or next_src_pinned.is_cuda
            or not next_src_pinned.is_contiguous()):
        raise ValueError(f"{fn}: next_dst must be a contiguous device tensor and "
                         "next_src_pinned a contiguous pinned host tensor of the same byte size")
    return next_dst.data_ptr(), next_src_pinned.data_ptr(), nbytes


def paged_attention_decode_shared_prefix(out, q, k_cache, v_cache, block_tables, context_lens,
                                         max_context_len: int, scale: float, members,
                                         member_flag, prefix_tokens: int, workspace=None,
                                         stream=None, seq_order=None) -> None:
    """``paged_attention_decode`` with a first partition of ``prefix_tokens``
    tokens (then partitions of max(2048, prefix_tokens)): the shared prefix
    of the sequences in ``members`` (device int32; their tables start with
    the same blocks) is computed once per tile of members.
    ``member_flag``: device int32 [num_seqs], nonzero for the members;
    ``workspace``: at least ``decode_workspace_bytes(..., prefix_tokens)``."""
    _shared_prefix("paged_attention_decode_shared_prefix", out, q, k_cache, v_cache,
                   block_tables, context_lens, max_context_len, scale, members, member_flag,
                   prefix_tokens, workspace, stream, seq_order, None)


def paged_attention_decode_shared_prefix_step(out, q, k_cache, v_cache, block_tables,
                                              context_lens, max_context_len: int, scale: float,
                                              members, member_flag, prefix_tokens: int,
                                              next_dst, next_src_pinned, workspace=None,
                                              stream=None, seq_order=None) -> None:
    """``paged_attention_decode_shared_prefix`` and, in the same launch, a
    copy of the pinned host tensor ``next_src_pinned`` into the device
    tensor ``next_dst`` (the next step's index arrays; equal byte sizes,
    multiples of 16)."""
    fn = "paged_attention_decode_shared_prefix_step"
    _shared_prefix(fn, out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                   scale, members, member_flag, prefix_tokens, workspace, stream, seq_order,
                   _next_upload(next_dst, next_src_pinned, fn))


def _shared_prefix(fn, out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                   scale, members, member_flag, prefix_tokens, workspace, stream, seq_order,
                   upload):
    B, Hq = q.shape[0], q.shape[1]
    idx = _decode_indices(block_tables, context_lens, seq_order, B, fn)
    M = members.numel() if members is not None else 0
    mp = _index_ptr(members, M, "members", fn) if M else None
    fp = _index_ptr(member_flag, B, "member_flag", fn) if M else None
    (N, bs, Hkv, D), dt = _caches(k_cache, v_cache, fn)
    qp, op = _q_out(q, out, (B, Hq, D), k_cache.dtype, fn)
    ws_ptr, ws_bytes = _workspace(workspace, fn)
    common = (op, qp, k_cache.data_ptr(), v_cache.data_ptr(), idx[0], block_tables.shape[1],
              idx[1], idx[2], int(max_context_len), B, Hq, Hkv, D, bs, N, float(scale), mp, fp, M,
              int(prefix_tokens), ws_ptr, ws_bytes)
    if upload is None:
        _check(lib.pkv_paged_attention_decode_shared_prefix(*common, dt, _stream_ptr(stream)), fn)
    else:
        _check(lib.pkv_paged_attention_decode_shared_prefix_step(
            *common, *upload, dt, _stream_ptr(stream)), fn)


def paged_attention_decode_write(out, q, new_key, new_value, k_cache, v_cache, block_tables,
                                 context_lens, max_context_len: int, scale: float,
                                 partition_size: int = PARTITION_AUTO, workspace=None,
                                 stream=None, seq_order=None) -> None:
    """The decode step in one launch: sequence b's new token (its last
    position, ``context_lens[b] - 1``) gets ``new_key[b]`` / ``new_value[b]``
    (``[B, Hkv, D]``, rows may be strided) written into the caches at the slot
    its block table gives, then ``paged_attention_decode``."""
    fn = "paged_attention_decode_write"
    B, Hq = q.shape[0], q.shape[1]
    idx = _decode_indices(block_tables, context_lens, seq_order, B, fn)
    (N, bs, Hkv, D), dt = _caches(k_cache, v_cache, fn)
    qp, op = _q_out(q, out, (B, Hq, D), k_cache.dtype, fn)
    kp = _dense_ptr(new_key, (B, Hkv, D), k_cache.dtype, "new_key", fn, rows=True)
    vp = _dense_ptr(new_value, (B, Hkv, D), k_cache.dtype, "new_value", fn, rows=True)
    ws_ptr, ws_bytes = _workspace(workspace, fn)
    _check(lib.pkv_paged_attention_decode_write(
        op, qp, kp, vp, new_key.stride(0) if B else Hkv * D,
        new_value.stride(0) if B else Hkv * D, k_cache.data_ptr(), v_cache.data_ptr(), idx[0],
        block_tables.shape[1], idx[1], idx[2], int(max_context_len), B, Hq, Hkv, D, bs, N,
        float(scale), int(partition_size), ws_ptr, ws_bytes, dt, _stream_ptr(stream)), fn)


def paged_attention_decode_step(out, q, new_key, new_value, k_cache, v_cache, block_tables,
                                context_lens, max_context_len: int, scale: float, next_dst,
                                next_src_pinned, partition_size: int = PARTITION_AUTO,
                                workspace=None, stream=None, seq_order=None) -> None:
    """``paged_attention_decode_write`` and, in the same launch, a copy of
    the pinned host tensor ``next_src_pinned`` into the device tensor
    ``next_dst`` (the next step's index arrays; equal byte sizes, multiples
    of 16).  ``new_key`` and ``new_value`` both None: a step without new
    tokens (``paged_attention_decode`` plus the upload)."""
    fn = "paged_attention_decode_step"
    B, Hq = q.shape[0], q.shape[1]
    idx = _decode_indices(block_tables, context_lens, seq_order, B, fn)
    (N, bs, Hkv, D), dt = _caches(k_cache, v_cache, fn)
    qp, op = _q_out(q, out, (B, Hq, D), k_cache.dtype, fn)
    if new_key is None and new_value is None:
        kp = vp = None
        ks = vs = 0
    else:
        if new_key is None or new_value is None:
            raise ValueError(f"{fn}: new_key and new_value are both tensors or both None")
        kp = _dense_ptr(new_key, (B, Hkv, D), k_cache.dtype, "new_key", fn, rows=True)
        vp = _dense_ptr(new_value, (B, Hkv, D), k_cache.dtype, "new_value", fn, rows=True)
        ks = new_key.stride(0) if B else Hkv * D
        vs = new_value.stride(0) if B else Hkv * D
    nd, ns, nbytes = _next_upload(next_dst, next_src_pinned, fn)
    ws_ptr, ws_bytes = _workspace(workspace, fn)
    _check(lib.pkv_paged_attention_decode_step(
        op, qp, kp, vp, ks, vs, k_cache.data_ptr(), v_cache.data_ptr(), idx[0],
        block_tables.shape[1], idx[1], idx[2], int(max_context_len), B, Hq, Hkv, D, bs, N,
        float(scale), int(partition_size), ws_ptr, ws_bytes, nd, ns, nbytes, dt,
        _stream_ptr(stream)), fn)


def upload_pinned(dst, src_pinned, stream=None) -> None:
    """Copy a pinned host tensor into a device tensor with a GPU kernel on the
    stream (never blocks the host); sizes must match, multiples of 16 bytes."""
    n = src_pinned.numel() * src_pinned.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("upload_pinned: size mismatch")
    if not dst.is_cuda or not dst.is_contiguous():
        raise ValueError("upload_pinned: dst must be a contiguous device tensor")
    if src_pinned.is_cuda or not src_pinned.is_contiguous():
        raise ValueError("upload_pinned: src must be a contiguous pinned host tensor")
    _check(lib.pkv_upload_pinned(dst.data_ptr(), src_pinned.data_ptr(), n, _stream_ptr(stream)),
           "upload_pinned")


def set_decode_path(path: int) -> None:
    """Process-wide decode kernel choice: PATH_AUTO, PATH_VALU or PATH_MFMA."""
    _check(lib.pkv_set_decode_path(int(path)), "set_decode_path")


def get_decode_path() -> int:
    return int(lib.pkv_get_decode_path())


def prefill_workspace_bytes(total_queries, num_q_heads, head_dim, max_context_len,
                            partition_size=PARTITION_AUTO) -> int:
    return int(lib.pkv_prefill_workspace_bytes(total_queries, num_q_heads, head_dim,
                                               max_context_len, partition_size))


def prefill_partition_size(num_seqs, max_queries_per_seq, num_q_heads, num_kv_heads,
                           max_context_len, partition_size=PARTITION_AUTO) -> int:
    """Partition size a prefill call uses (AUTO resolved); 0 = single pass."""
    return int(lib.pkv_prefill_partition_size(num_seqs, max_queries_per_seq, num_q_heads,
                                              num_kv_heads, max_context_len, partition_size))


def paged_attention_prefill(out, q, query_start, max_queries_per_seq: int, k_cache, v_cache,
                            block_tables, context_lens, max_context_len: int, scale: float,
                            partition_size: int = PARTITION_AUTO, workspace=None, stream=None,
                            seq_order=None) -> None:
    """Chunked prefill: query rows ``query_start[b] .. query_start[b+1]-1`` of
    ``q [T, Hq, D]`` are the last tokens of sequence ``b`` and attend causally
    to its paged context.  ``query_start``: device int32 ``[B + 1]``."""
    fn = "paged_attention_prefill"
    T, Hq = q.shape[0], q.shape[1]
    B = context_lens.shape[0]
    qs = _index_ptr(query_start, B + 1, "query_start", fn)
    idx = _decode_indices(block_tables, context_lens, seq_order, B, fn)
    (N, bs, Hkv, D), dt = _caches(k_cache, v_cache, fn)
    qp, op = _q_out(q, out, (T, Hq, D), k_cache.dtype, fn)
    ws_ptr, ws_bytes = _workspace(workspace, fn)
    _check(lib.pkv_paged_attention_prefill(
        op, qp, qs, T, int(max_queries_per_seq), k_cache.data_ptr(), v_cache.data_ptr(), idx[0],
        block_tables.shape[1], idx[1], idx[2], int(max_context_len), B, Hq, Hkv, D, bs, N,
        float(scale), int(partition_size), ws_ptr, ws_bytes, dt, _stream_ptr(stream)), fn)


def copy_blocks(k_cache, v_cache, pairs, stream=None) -> None:
    """``cache[dst] = cache[src]`` for each row ``(src, dst)`` of int64 ``pairs [P, 2]``."""
    pp = _index_ptr(pairs, 0, "pairs", "copy_blocks", wide=True, cols=2)
    (N, bs, Hkv, D), dt = _caches(k_cache, v_cache, "copy_blocks")
    _check(lib.pkv_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), pp, pairs.shape[0], N, bs,
                               Hkv, D, dt, _stream_ptr(stream)), "copy_blocks")


def swap_blocks(k_cache, v_cache, k_host, v_host, pairs, direction: int, stream=None) -> None:
    """Swap copy between the device caches and the pinned host pools
    ``[Nh, bs, Hkv, D]`` (torch CPU tensors from ``pin_memory()``):
    SWAP_OUT copies device block ``src`` to host block ``dst`` for each row of
    ``pairs`` (device int64 ``[P, 2]``), SWAP_IN host ``src`` to device ``dst``."""
    pp = _index_ptr(pairs, 0, "pairs", "swap_blocks", wide=True, cols=2)
    (N, bs, Hkv, D), dt = _caches(k_cache, v_cache, "swap_blocks")
    Nh = k_host.shape[0]
    if tuple(k_host.shape[1:]) != (bs, Hkv, D) or k_host.shape != v_host.shape:
        raise ValueError("host pools must be [num_host_blocks, block_size, Hkv, D]")
    if k_host.dtype != k_cache.dtype or v_host.dtype != k_cache.dtype:
        raise TypeError("host pools must have the cache dtype")
    if (k_host.is_cuda or v_host.is_cuda or not k_host.is_contiguous()
            or not v_host.is_contiguous()):
        raise ValueError("swap_blocks: host pools must be contiguous pinned host tensors")
    _check(lib.pkv_swap_blocks(k_cache.data_ptr(), v_cache.data_ptr(), k_host.data_ptr(),
                               v_host.data_ptr(), pp, pairs.shape[0], N, Nh, bs, Hkv, D, dt,
                               int(direction), _stream_ptr(stream)), "swap_blocks")


# ------------------------------------------------------------------ host checks
def blocks_for_budget(nbytes: int, num_layers: int, block_size: int, num_kv_heads: int,
                      head_dim: int, dtype: int = BF16) -> int:
    """Cache blocks (K and V of every layer) that ``nbytes`` of memory hold;
    -1 for invalid sizes."""
    return int(lib.pkv_blocks_for_budget(int(nbytes), num_layers, block_size, num_kv_heads,
                                         head_dim, dtype))


def _host_i32(a, what: str):
    """A contiguous host int32 copy of ``a`` (numpy or torch) and its pointer."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    arr = np.ascontiguousarray(a, dtype=np.int32)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def validate_decode_inputs(block_tables, context_lens, max_context_len: int, block_size: int,
                           num_blocks: int, seq_order=None, members=None, member_flag=None,
                           prefix_tokens: int = 0) -> None:
    """Debug check of a decode call's index arrays on the host: every table
    entry a context reads lies in the pool, every length within
    ``max_context_len`` and the table width, the launch order is a
    permutation, and shared-prefix members share their first
    ``prefix_tokens`` tokens' blocks.  Raises ``PkvError`` (INVALID_ARG)
    naming the first bad entry.  Device tensors are copied to the host."""
    tb, tp = _host_i32(block_tables, "block_tables")
    if tb.ndim != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    cx, cp = _host_i32(context_lens, "context_lens")
    if cx.shape != (tb.shape[0],):
        raise ValueError("context_lens must have one entry per table row")
    keep = [tb, cx]
    op = mp = fp = None
    if seq_order is not None:
        o, op = _host_i32(seq_order, "seq_order")
        if o.shape != cx.shape:
            raise ValueError("seq_order must have one entry per sequence")
        keep.append(o)
    nm = 0
    if members is not None:
        m, mp = _host_i32(members, "members")
        f, fp = _host_i32(member_flag, "member_flag")
        if f.shape != cx.shape:
            raise ValueError("member_flag must have one entry per sequence")
        keep += [m, f]
        nm = m.size
    _check(lib.pkv_validate_decode_inputs(tp, tb.shape[0], tb.shape[1], cp, op,
                                          int(max_context_len), block_size, num_blocks, mp, fp,
                                          nm, int(prefix_tokens)), "validate_decode_inputs")


# ------------------------------------------------------------------ allocator
class Allocator:
    """Host block allocator (C++); see ``pkv_allocator_*`` in ``include/pkv.h``."""

    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        h = ctypes.c_void_p()
        fo = None
        if free_order is not None:
            self._fo = np.ascontiguousarray(free_order, dtype=np.int32)
            if self._fo.shape != (num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
            fo = self._fo.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        _check(lib.pkv_allocator_create(num_blocks, block_size, fo, ctypes.byref(h)),
               "allocator_create")
        self._h = h
        self._destroy = lib.pkv_allocator_destroy  # still callable at interpreter exit
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add(self, seq: int) -> None:
        _check(lib.pkv_seq_add(self._h, seq), "seq_add")

    def fork_prefix(self, src: int, dst: int, num_tokens: int) -> None:
        _check(lib.pkv_seq_fork_prefix(self._h, src, dst, num_tokens), "seq_fork_prefix")

    def append(self, seq: int, n: int) -> np.ndarray:
        out = np.empty(max(n, 0), dtype=np.int64)
        _check(lib.pkv_seq_append(self._h, seq, n,
                                  out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))), "seq_append")
        return out

    def append_tokens(self, seqs: Sequence[int], counts: Sequence[int],
                      out: Optional[np.ndarray] = None) -> np.ndarray:
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        c = np.ascontiguousarray(counts, dtype=np.int32)
        total = int(c.sum()) if len(c) else 0
        if out is None:
            out = np.empty(total, dtype=np.int64)
        elif out.dtype != np.int64 or out.size < total or not out.flags.c_contiguous:
            raise ValueError("out must be a contiguous int64 array large enough")
        _check(lib.pkv_append_tokens(self._h, s.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(s),
                                     out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))),
               "append_tokens")
        return out[:total]

    def append_cow(self, seqs: Sequence[int], counts: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
        """Copy-on-write append: returns (slots, copy pairs int64 [P, 2]); copy
        the pairs' blocks (``copy_blocks``) before writing the new tokens."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        c = np.ascontiguousarray(counts, dtype=np.int32)
        slots = np.empty(int(c.sum()) if len(c) else 0, dtype=np.int64)
        pairs = np.empty((max(len(s), 1), 2), dtype=np.int64)
        npairs = ctypes.c_int32(0)
        _check(lib.pkv_append_tokens_cow(self._h, s.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                         c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(s),
                                         slots.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                         pairs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                         len(pairs), ctypes.byref(npairs)), "append_tokens_cow")
        return slots, pairs[: npairs.value].copy()

    def free(self, seq: int) -> None:
        _check(lib.pkv_seq_free(self._h, seq), "seq_free")

    def set_host_pool(self, num_host_blocks: int,
                      host_free_order: Optional[Sequence[int]] = None) -> None:
        fo = None
        if host_free_order is not None:
            self._hfo = np.ascontiguousarray(host_free_order, dtype=np.int32)
            if self._hfo.shape != (num_host_blocks,):
                raise ValueError("host_free_order must have num_host_blocks entries")
            fo = self._hfo.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        _check(lib.pkv_allocator_set_host_pool(self._h, num_host_blocks, fo), "set_host_pool")
        self.num_host_blocks = num_host_blocks

    def _move(self, fn, name: str, seqs: Sequence[int]) -> np.ndarray:
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        room = sum(max(self.num_blocks_of(int(x)), 0) for x in s)
        pairs = np.empty((max(room, 1), 2), dtype=np.int64)
        npairs = ctypes.c_int32(0)
        _check(fn(self._h, s.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(s),
                  pairs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(pairs),
                  ctypes.byref(npairs)), name)
        return pairs[: npairs.value].copy()

    def swap_out(self, seqs: Sequence[int]) -> np.ndarray:
        """Move the sequences to host blocks; returns the (device, host) block
        pairs int64 [P, 2] to copy with ``swap_blocks(..., SWAP_OUT)``."""
        return self._move(lib.pkv_swap_out, "swap_out", seqs)

    def swap_in(self, seqs: Sequence[int]) -> np.ndarray:
        """Move swapped-out sequences back to fresh device blocks; returns the
        (host, device) pairs to copy with ``swap_blocks(..., SWAP_IN)``."""
        return self._move(lib.pkv_swap_in, "swap_in", seqs)

    def enable_prefix_cache(self) -> None:
        _check(lib.pkv_allocator_enable_prefix_cache(self._h), "enable_prefix_cache")

    def add_prompt(self, seq: int, tokens: Sequence[int],
                   slots_out: Optional[np.ndarray] = None) -> Tuple[np.ndarray, int]:
        """New sequence for a prompt; returns (slots of the tokens after the
        shared cached prefix, number of shared tokens)."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        out = slots_out if slots_out is not None else np.empty(len(t), dtype=np.int64)
        if out.dtype != np.int64 or out.size < len(t) or not out.flags.c_contiguous:
            raise ValueError("slots_out must be a contiguous int64 array of len(tokens)")
        cached = ctypes.c_int32(0)
        _check(lib.pkv_seq_add_prompt(self._h, seq, t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      len(t), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                      ctypes.byref(cached)), "seq_add_prompt")
        return out[: len(t) - cached.value], int(cached.value)

    def prefix_cache_stats(self) -> Tuple[int, int, int]:
        """(full-block lookups, hits, blocks holding a cached prefix)."""
        lk, ht, nc = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int32(0)
        _check(lib.pkv_prefix_cache_stats(self._h, ctypes.byref(lk), ctypes.byref(ht),
                                          ctypes.byref(nc)), "prefix_cache_stats")
        return int(lk.value), int(ht.value), int(nc.value)

    def is_swapped(self, seq: int) -> int:
        return int(lib.pkv_seq_is_swapped(self._h, seq))

    def num_free_host_blocks(self) -> int:
        return int(lib.pkv_num_free_host_blocks(self._h))

    def host_block_refcount(self, block: int) -> int:
        return int(lib.pkv_host_block_refcount(self._h, block))

    def build_block_tables(self, seqs: Sequence[int], max_blocks: int, pad: int = -1,
                           tables_out: Optional[np.ndarray] = None,
                           ctx_out: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        t = tables_out if tables_out is not None else np.empty((len(s), max_blocks), np.int32)
        c = ctx_out if ctx_out is not None else np.empty(len(s), np.int32)
        if t.dtype != np.int32 or t.shape != (len(s), max_blocks) or not t.flags.c_contiguous:
            raise ValueError("tables_out must be a contiguous int32 [num_seqs, max_blocks]")
        _check(lib.pkv_build_block_tables(self._h, s.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                          len(s), max_blocks, pad,
                                          t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                          c.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
               "build_block_tables")
        return t, c

    def decode_step_prepare(self, seqs: np.ndarray, max_blocks: int, slots_out: np.ndarray,
                            tables_out: np.ndarray, ctx_out: np.ndarray, pad: int = -1,
                            order_out: Optional[np.ndarray] = None) -> int:
        """Grow every sequence in ``seqs`` (int64) by one token and write the
        new slots, the tables, context lengths and (optionally) the
        longest-first launch order into the given host arrays (contiguous
        int64 / int32 / int32 / int32); returns the longest context."""
        mx = ctypes.c_int32(0)
        po = ctypes.POINTER(ctypes.c_int32)
        _check(lib.pkv_decode_step_prepare(
            self._h, seqs.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(seqs), max_blocks,
            pad, slots_out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            tables_out.ctypes.data_as(po), ctx_out.ctypes.data_as(po), ctypes.byref(mx),
            order_out.ctypes.data_as(po) if order_out is not None else None),
            "decode_step_prepare")
        return int(mx.value)

    def shared_prefix_members(self, seqs: Sequence[int],
                              prefix_tokens: int) -> Tuple[np.ndarray, np.ndarray]:
        """Batch positions of the sequences of ``seqs`` that share the blocks
        of a ``prefix_tokens``-token prefix (the largest such group), and the
        per-position flag: the ``members`` / ``member_flag`` arguments of
        ``paged_attention_decode_shared_prefix``, int32."""
        s = np.ascontiguousarray(seqs, dtype=np.int64)
        members = np.empty(max(len(s), 1), dtype=np.int32)
        flag = np.empty(max(len(s), 1), dtype=np.int32)
        n = ctypes.c_int32(0)
        po = ctypes.POINTER(ctypes.c_int32)
        _check(lib.pkv_shared_prefix_members(self._h, s.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                             len(s), int(prefix_tokens), members.ctypes.data_as(po),
                                             flag.ctypes.data_as(po), ctypes.byref(n)),
               "shared_prefix_members")
        return members[: n.value].copy(), flag[: len(s)].copy()

    def num_free_blocks(self) -> int:
        return int(lib.pkv_num_free_blocks(self._h))

    def block_refcount(self, block: int) -> int:
        return int(lib.pkv_block_refcount(self._h, block))

    def context_len(self, seq: int) -> int:
        return int(lib.pkv_seq_context_len(self._h, seq))

    def num_blocks_of(self, seq: int) -> int:
        return int(lib.pkv_seq_num_blocks(self._h, seq))

    def replay(self, ops: Iterable[tuple]) -> None:
        """Run a workload's op list (``add`` / ``append`` / ``fork``)."""
        for op in ops:
            if op[0] == "add":
                self.add(op[1])
            elif op[0] == "append":
                self.append(op[1], op[2])
            elif op[0] == "fork":
                self.fork_prefix(op[1], op[2], op[3])
            else:
                raise ValueError(op)
