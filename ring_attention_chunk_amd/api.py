"""Thin Python binding of the C ABI (ctypes): argument marshalling only.

Every step of the computation runs in the HIP library; this module checks
tensor shapes, fills the C descriptor structs, allocates outputs with torch
(device memory is torch's) and passes torch's current stream. There is no
fallback: if the library is missing or no GPU is present, calls raise.

The three calls keep the names of the exercise page
"systems-distributed-ring-attention-online-softmax" (problem statement):
``attention_chunk_stats``, ``merge_chunk_stats`` and ``ring_attention``.
"""

from __future__ import annotations

import ctypes
import functools
import math
import os
from typing import List, Optional, Sequence, Tuple, Union

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libring_attention_chunk.so")

RA_F32, RA_BF16 = 0, 1

# exported symbols, as declared in include/ring_attention_chunk.h
EXPORTS = (
    "ra_attention_chunk_stats",
    "ra_chunk_stats_workspace_bytes",
    "ra_merge_chunk_stats",
    "ra_ring_workspace_bytes",
    "ra_ring_attention",
    "ra_ring_attention_noalloc",
    "ra_block_sparse_workspace_bytes",
    "ra_ring_attention_block_sparse",
    "ra_ring_backward_workspace_bytes",
    "ra_ring_attention_backward",
    "ra_kernel_timer",
    "ra_kernel_timer_read",
    "ra_status_string",
    "ra_last_error",
)


class KVChunk(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("len", ctypes.c_int64),
        ("global_offset", ctypes.c_int64),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("stride_s", ctypes.c_int64),
        ("pos_stride", ctypes.c_int64),
    ]


class QSegment(ctypes.Structure):
    _fields_ = [("len", ctypes.c_int64), ("global_offset", ctypes.c_int64), ("pos_stride", ctypes.c_int64)]


class RingAttentionError(RuntimeError):
    pass


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RingAttentionError(
            f"HIP library not found at {path}; build it with "
            "`python -m ring_attention_chunk_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.ra_attention_chunk_stats.argtypes = [i32, i32, i32, i32, i32, vp, i64, ctypes.POINTER(KVChunk), f32,
                                             vp, vp, vp, vp, sz, vp]
    lib.ra_attention_chunk_stats.restype = i32
    lib.ra_chunk_stats_workspace_bytes.argtypes = [i32, i32, i32, i64, i64]
    lib.ra_chunk_stats_workspace_bytes.restype = sz
    lib.ra_merge_chunk_stats.argtypes = [i64, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.ra_merge_chunk_stats.restype = i32
    lib.ra_ring_workspace_bytes.argtypes = [i32, i32, i32, i64, i64, i32, i32]
    lib.ra_ring_workspace_bytes.restype = sz
    lib.ra_ring_attention.argtypes = [i32, i32, i32, i32, i32, vp, ctypes.POINTER(QSegment), i32,
                                      ctypes.POINTER(KVChunk), i32, i32, f32, vp, sz, vp, vp, vp]
    lib.ra_ring_attention.restype = i32
    lib.ra_ring_attention_noalloc.argtypes = [i32, i32, i32, i32, i32, vp, ctypes.POINTER(QSegment), i32,
                                              ctypes.POINTER(KVChunk), i32, i32, f32, vp, vp, vp]
    lib.ra_ring_attention_noalloc.restype = i32
    lib.ra_block_sparse_workspace_bytes.argtypes = [i32, i32, i32, i64, i64, i32, i32, i64, i64]
    lib.ra_block_sparse_workspace_bytes.restype = sz
    lib.ra_ring_attention_block_sparse.argtypes = [i32, i32, i32, i32, i32, vp, ctypes.POINTER(QSegment), i32,
                                                   ctypes.POINTER(KVChunk), i32, i32, f32, vp, i64, i64, i64, i64, vp,
                                                   sz, vp, vp, vp]
    lib.ra_ring_attention_block_sparse.restype = i32
    lib.ra_ring_backward_workspace_bytes.argtypes = [i32, i32, i32, i64, i64, i32, i32]
    lib.ra_ring_backward_workspace_bytes.restype = sz
    lib.ra_ring_attention_backward.argtypes = [i32, i32, i32, i32, i32, vp, ctypes.POINTER(QSegment), i32,
                                               ctypes.POINTER(KVChunk), i32, i32, f32, vp, vp, vp, vp, sz, vp, vp,
                                               vp, vp]
    lib.ra_ring_attention_backward.restype = i32
    lib.ra_kernel_timer.argtypes = [i32]
    lib.ra_kernel_timer.restype = i32
    lib.ra_kernel_timer_read.argtypes = [ctypes.POINTER(f32), ctypes.POINTER(i32)]
    lib.ra_kernel_timer_read.restype = i32
    lib.ra_status_string.argtypes = [i32]
    lib.ra_status_string.restype = ctypes.c_char_p
    lib.ra_last_error.argtypes = []
    lib.ra_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(lib, status: int, what: str):
    if status != 0:
        msg = lib.ra_last_error().decode()
        name = lib.ra_status_string(status).decode()
        raise RingAttentionError(f"{what}: {name} ({status}): {msg}")


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise RingAttentionError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _require_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise RingAttentionError("tensors must live on the GPU (no CPU path exists)")


def _chunk_desc(k, v, offset: int, batch: int, kv_heads: int, head_dim: int, pos_stride: int = 1) -> KVChunk:
    if k.dim() != 4 or v.dim() != 4:
        raise RingAttentionError("key/value chunks must be [batch, kv_heads, len, head_dim]")
    if tuple(k.shape) != tuple(v.shape):
        raise RingAttentionError(f"key chunk {tuple(k.shape)} and value chunk {tuple(v.shape)} differ")
    if k.shape[0] != batch or k.shape[1] != kv_heads or k.shape[3] != head_dim:
        raise RingAttentionError(f"chunk shape {tuple(k.shape)} does not match batch={batch}, "
                                 f"kv_heads={kv_heads}, head_dim={head_dim}")
    if k.stride() != v.stride():
        raise RingAttentionError("key and value chunks must share strides")
    if k.shape[2] > 0 and k.stride(3) != 1:
        raise RingAttentionError("the head_dim axis of a chunk must be contiguous")
    sb, sh, ss, _ = k.stride()
    if k.shape[2] <= 1:
        ss = max(ss, head_dim)
    return KVChunk(k.data_ptr(), v.data_ptr(), int(k.shape[2]), int(offset), int(sb), int(sh), int(ss),
                   int(pos_stride))


@functools.lru_cache(maxsize=256)
def _stats_workspace_bytes(B: int, Hq: int, d: int, Lq: int, Lc: int) -> int:
    return int(load_library().ra_chunk_stats_workspace_bytes(B, Hq, d, Lq, Lc))


def attention_chunk_stats(query, key_chunk, value_chunk, scale: Optional[float] = None, workspace=None):
    """Statistics of one chunk: ``(u, l, m)`` (un-normalised numerator, denominator, row max).

    query [B, Hq, Lq, d]; key_chunk, value_chunk [B, Hkv, Lc, d] (bf16 or fp32, on the GPU).
    Returns fp32 tensors u [B, Hq, Lq, d], l and m [B, Hq, Lq]. When the query rows alone cannot
    fill the GPU, a device workspace for key-range partials is allocated (torch) unless one is
    given.
    """
    torch = _torch()
    lib = load_library()
    _require_gpu(query, key_chunk, value_chunk)
    if query.dim() != 4:
        raise RingAttentionError("query must be [batch, q_heads, q_len, head_dim]")
    if key_chunk.dtype != query.dtype or value_chunk.dtype != query.dtype:
        raise RingAttentionError("query, key and value must share a dtype")
    q = query.contiguous()
    B, Hq, Lq, d = q.shape
    Hkv = key_chunk.shape[1] if key_chunk.dim() == 4 else 0
    desc = _chunk_desc(key_chunk, value_chunk, 0, B, Hkv, d)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    u = torch.empty((B, Hq, Lq, d), dtype=torch.float32, device=q.device)
    l = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    m = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    need = _stats_workspace_bytes(B, Hq, d, Lq, int(key_chunk.shape[2]))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() if workspace is not None else 0
    st = lib.ra_attention_chunk_stats(_dtype_code(q), B, Hq, Hkv, d, q.data_ptr(), Lq, ctypes.byref(desc),
                                      float(scale), u.data_ptr(), l.data_ptr(), m.data_ptr(), ws_ptr, ws_len,
                                      _stream(q))
    _check(lib, st, "attention_chunk_stats")
    return u, l, m


def merge_chunk_stats(acc, chunk, inplace: bool = False):
    """Merge ``chunk = (u, l, m)`` into ``acc = (u, l, m)`` by the rescale-to-shared-max rule.

    Returns the merged triple. With ``inplace=True`` the accumulator tensors
    are overwritten and returned; otherwise new tensors are returned.
    """
    lib = load_library()
    au, al, am = acc
    bu, bl, bm = chunk
    _require_gpu(au, al, am, bu, bl, bm)
    for t in (au, al, am, bu, bl, bm):
        if t.dtype != _torch().float32:
            raise RingAttentionError("statistics are fp32 tensors")
    if au.shape != bu.shape or al.shape != bl.shape or am.shape != bm.shape or al.shape != am.shape:
        raise RingAttentionError("accumulator and chunk statistics differ in shape")
    if tuple(au.shape[:-1]) != tuple(al.shape):
        raise RingAttentionError("u must be l's shape plus a trailing head_dim axis")
    if not inplace:
        # fresh row-major copies: the kernel reads and writes u as [rows, head_dim]
        au, al, am = (t.clone(memory_format=_torch().contiguous_format) for t in (au, al, am))
    elif not (au.is_contiguous() and al.is_contiguous() and am.is_contiguous()):
        raise RingAttentionError("in-place merge needs contiguous accumulator tensors")
    bu, bl, bm = bu.contiguous(), bl.contiguous(), bm.contiguous()
    d = au.shape[-1]
    rows = al.numel()
    st = lib.ra_merge_chunk_stats(rows, d, au.data_ptr(), al.data_ptr(), am.data_ptr(), bu.data_ptr(),
                                  bl.data_ptr(), bm.data_ptr(), _stream(au))
    _check(lib, st, "merge_chunk_stats")
    return au, al, am


QOffset = Union[int, Sequence[Union[Tuple[int, int], Tuple[int, int, int]]]]


def kernel_timer(enable: bool) -> None:
    """ra_kernel_timer: start (clearing earlier records) or stop recording the device time of the
    attention kernel of each call."""
    lib = load_library()
    _check(lib, lib.ra_kernel_timer(1 if enable else 0), "kernel_timer")


def kernel_timer_read():
    """ra_kernel_timer_read: (total milliseconds, number of recorded calls), clearing the records."""
    lib = load_library()
    tot, n = ctypes.c_float(0.0), ctypes.c_int(0)
    _check(lib, lib.ra_kernel_timer_read(ctypes.byref(tot), ctypes.byref(n)), "kernel_timer_read")
    return float(tot.value), int(n.value)


def workspace_bytes(query_shape, key_lengths, n_q_segments: int = 1) -> int:
    """Bytes of device workspace ``ring_attention`` needs for this shape."""
    B, Hq, Lq, d = query_shape
    return int(load_library().ra_ring_workspace_bytes(B, Hq, d, Lq, int(sum(key_lengths)), len(key_lengths),
                                                      n_q_segments))


def backward_workspace_bytes(query_shape, key_lengths, n_q_segments: int = 1) -> int:
    """Bytes of device workspace ``ring_attention_backward`` needs for this shape."""
    B, Hq, Lq, d = query_shape
    return int(load_library().ra_ring_backward_workspace_bytes(B, Hq, d, Lq, int(sum(key_lengths)),
                                                               len(key_lengths), n_q_segments))


def ring_attention(query, key_chunks: Sequence, value_chunks: Sequence, q_global_offset: QOffset = 0,
                   kv_global_offsets: Optional[Sequence[int]] = None, causal: bool = False,
                   scale: Optional[float] = None, return_lse: bool = False, workspace=None,
                   kv_position_strides: Optional[Sequence[int]] = None):
    """Attention of the local queries over all chunks, in list (ring) order, normalised once.

    ``q_global_offset`` is the global position of the first query (an int), or
    a list of ``(global_offset, length)`` runs covering the query rows (two
    runs for a paired early/late share), or ``(global_offset, length, step)``
    runs whose positions advance by ``step`` per row (a striped share).
    ``kv_global_offsets`` gives each chunk's first global position; by default
    chunks follow each other from 0. ``kv_position_strides`` gives each
    chunk's position step (default 1; P for a striped shard of P devices).
    Returns out [B, Hq, Lq, d] fp32 (and lse [B, Hq, Lq] if ``return_lse``).
    """
    torch = _torch()
    lib = load_library()
    Hkv, descs, n, segs, nseg = _marshal(query, key_chunks, value_chunks, q_global_offset, kv_global_offsets,
                                         kv_position_strides)
    q = query.contiguous()
    B, Hq, Lq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    total_keys = sum(int(k.shape[2]) for k in key_chunks)
    need = lib.ra_ring_workspace_bytes(B, Hq, d, Lq, total_keys, n, nseg)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace.numel() < need or workspace.data_ptr() % 256 != 0:
        raise RingAttentionError(f"workspace must hold {need} bytes at a 256-byte aligned address")
    out = torch.empty((B, Hq, Lq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device) if return_lse else None
    st = lib.ra_ring_attention(_dtype_code(q), B, Hq, Hkv, d, q.data_ptr(), segs, nseg, descs, n,
                               int(bool(causal)), float(scale), workspace.data_ptr(), workspace.numel(),
                               out.data_ptr(), lse.data_ptr() if lse is not None else None, _stream(q))
    _check(lib, st, "ring_attention")
    return (out, lse) if return_lse else out


def ring_attention_noalloc(query, key_chunks: Sequence, value_chunks: Sequence, q_global_offset: QOffset = 0,
                           kv_global_offsets: Optional[Sequence[int]] = None, causal: bool = False,
                           scale: Optional[float] = None, kv_position_strides: Optional[Sequence[int]] = None,
                           out=None, lse=None):
    """:func:`ring_attention` through ``ra_ring_attention_noalloc``: no workspace, no device allocation in the
    library (its tables and partials live in a per-GPU static array of ``RA_NOALLOC_SCRATCH_BYTES``).

    Pass ``out`` [B, Hq, Lq, d] fp32 (and optionally ``lse`` [B, Hq, Lq] fp32), contiguous, to make the whole
    call allocation-free; without them this wrapper allocates them with torch. Returns ``out`` (and
    ``lse`` when given). Calls that overlap on one GPU race on the shared array."""
    torch = _torch()
    lib = load_library()
    Hkv, descs, n, segs, nseg = _marshal(query, key_chunks, value_chunks, q_global_offset, kv_global_offsets,
                                         kv_position_strides)
    if not query.is_contiguous():
        raise RingAttentionError("the allocation-free call needs a contiguous query")
    B, Hq, Lq, d = query.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, Lq, d), dtype=torch.float32, device=query.device)
    for t, shape in ((out, (B, Hq, Lq, d)), (lse, (B, Hq, Lq))):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous()):
            raise RingAttentionError(f"outputs must be contiguous fp32 tensors of shape {shape}")
    st = lib.ra_ring_attention_noalloc(_dtype_code(query), B, Hq, Hkv, d, query.data_ptr(), segs, nseg, descs, n,
                                       int(bool(causal)), float(scale), out.data_ptr(),
                                       lse.data_ptr() if lse is not None else None, _stream(query))
    _check(lib, st, "ring_attention_noalloc")
    return (out, lse) if lse is not None else out


def ring_attention_block_sparse(query, key_chunks: Sequence, value_chunks: Sequence, block_mask, block_q: int,
                                block_k: int, q_global_offset: QOffset = 0,
                                kv_global_offsets: Optional[Sequence[int]] = None, causal: bool = False,
                                scale: Optional[float] = None, return_lse: bool = False, workspace=None,
                                kv_position_strides: Optional[Sequence[int]] = None):
    """:func:`ring_attention` restricted by a block mask over global positions.

    ``block_mask`` is a [n_qblocks, n_kblocks] bool or uint8 tensor on the GPU: a query at position p may see a
    key at position k when ``block_mask[p // block_q, k // block_k]`` (and, with ``causal``, k <= p). Block
    sizes are powers of two. Other arguments as for :func:`ring_attention`.
    """
    torch = _torch()
    lib = load_library()
    Hkv, descs, n, segs, nseg = _marshal(query, key_chunks, value_chunks, q_global_offset, kv_global_offsets,
                                         kv_position_strides)
    _require_gpu(block_mask)
    if block_mask.dim() != 2 or block_mask.dtype not in (torch.bool, torch.uint8):
        raise RingAttentionError("block_mask must be a 2-D bool or uint8 tensor")
    m = block_mask.to(torch.uint8).contiguous()
    q = query.contiguous()
    B, Hq, Lq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    total_keys = sum(int(k.shape[2]) for k in key_chunks)
    need = lib.ra_block_sparse_workspace_bytes(B, Hq, d, Lq, total_keys, n, nseg, int(m.shape[0]), int(m.shape[1]))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace.numel() < need or workspace.data_ptr() % 256 != 0:
        raise RingAttentionError(f"workspace must hold {need} bytes at a 256-byte aligned address")
    out = torch.empty((B, Hq, Lq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device) if return_lse else None
    st = lib.ra_ring_attention_block_sparse(_dtype_code(q), B, Hq, Hkv, d, q.data_ptr(), segs, nseg, descs, n,
                                            int(bool(causal)), float(scale), m.data_ptr(), int(m.shape[0]),
                                            int(m.shape[1]), int(block_q), int(block_k), workspace.data_ptr(),
                                            workspace.numel(), out.data_ptr(),
                                            lse.data_ptr() if lse is not None else None, _stream(q))
    _check(lib, st, "ring_attention_block_sparse")
    return (out, lse) if return_lse else out


def _marshal(query, key_chunks, value_chunks, q_global_offset, kv_global_offsets, kv_position_strides):
    """Shared argument checks of the ring calls: descriptors and query runs."""
    if len(key_chunks) != len(value_chunks):
        raise RingAttentionError("key_chunks and value_chunks differ in length")
    _require_gpu(query, *key_chunks, *value_chunks)
    if query.dim() != 4:
        raise RingAttentionError("query must be [batch, q_heads, q_len, head_dim]")
    B, Hq, Lq, d = query.shape
    for t in list(key_chunks) + list(value_chunks):
        if t.dtype != query.dtype:
            raise RingAttentionError("query, keys and values must share a dtype")
    if kv_global_offsets is None:
        kv_global_offsets, acc = [], 0
        for k in key_chunks:
            kv_global_offsets.append(acc)
            acc += int(k.shape[2])
    if len(kv_global_offsets) != len(key_chunks):
        raise RingAttentionError("one global offset per chunk is required")
    if kv_position_strides is None:
        kv_position_strides = [1] * len(key_chunks)
    if len(kv_position_strides) != len(key_chunks):
        raise RingAttentionError("one position stride per chunk is required")
    Hkv = int(key_chunks[0].shape[1]) if key_chunks else Hq
    n = len(key_chunks)
    descs = (KVChunk * max(n, 1))()
    for i, (k, v, off, ps) in enumerate(zip(key_chunks, value_chunks, kv_global_offsets, kv_position_strides)):
        descs[i] = _chunk_desc(k, v, off, B, Hkv, d, ps)
    if isinstance(q_global_offset, int):
        segs_py = [(int(q_global_offset), Lq, 1)]
    else:
        segs_py = [(int(g[0]), int(g[1]), int(g[2]) if len(g) > 2 else 1) for g in q_global_offset]
    if sum(g[1] for g in segs_py) != Lq:
        raise RingAttentionError(f"query segments cover {sum(g[1] for g in segs_py)} rows, query has {Lq}")
    segs = (QSegment * len(segs_py))(*[QSegment(n_, o, ps) for o, n_, ps in segs_py])
    return Hkv, descs, n, segs, len(segs_py)


def ring_attention_backward(query, key_chunks: Sequence, value_chunks: Sequence, out, lse, dout,
                            q_global_offset: QOffset = 0, kv_global_offsets: Optional[Sequence[int]] = None,
                            causal: bool = False, scale: Optional[float] = None,
                            kv_position_strides: Optional[Sequence[int]] = None, workspace=None):
    """Gradients of :func:`ring_attention` for this share: ``(dq, dk_chunks, dv_chunks)``.

    ``out`` and ``lse`` are what ``ring_attention(..., return_lse=True)``
    returned for the same inputs; ``dout`` is the gradient of the output (same
    dtype as the query; bf16 only). ``dq`` is [B, Hq, Lq, d] fp32; ``dk_chunks``
    and ``dv_chunks`` hold, per chunk, this share's contribution to that
    chunk's key and value gradients, [B, Hkv, len, d] fp32 each (views of one
    buffer in list order).
    """
    torch = _torch()
    lib = load_library()
    Hkv, descs, n, segs, nseg = _marshal(query, key_chunks, value_chunks, q_global_offset, kv_global_offsets,
                                         kv_position_strides)
    q = query.contiguous()
    B, Hq, Lq, d = q.shape
    _require_gpu(out, lse, dout)
    if dout.dtype != q.dtype or tuple(dout.shape) != tuple(q.shape):
        raise RingAttentionError("dout must have the query's shape and dtype")
    if out.dtype != torch.float32 or tuple(out.shape) != tuple(q.shape):
        raise RingAttentionError("out must be the fp32 output of ring_attention")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Lq):
        raise RingAttentionError("lse must be the fp32 [B, Hq, Lq] log-sum-exp of ring_attention")
    do, o, ls = dout.contiguous(), out.contiguous(), lse.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = [int(k.shape[2]) for k in key_chunks]
    total = sum(lens)
    need = lib.ra_ring_backward_workspace_bytes(B, Hq, d, Lq, total, n, nseg)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace.numel() < need or workspace.data_ptr() % 256 != 0:
        raise RingAttentionError(f"workspace must hold {need} bytes at a 256-byte aligned address")
    dq = torch.empty((B, Hq, Lq, d), dtype=torch.float32, device=q.device)
    dk = torch.empty((B, Hkv, total, d), dtype=torch.float32, device=q.device)
    dv = torch.empty((B, Hkv, total, d), dtype=torch.float32, device=q.device)
    st = lib.ra_ring_attention_backward(_dtype_code(q), B, Hq, Hkv, d, q.data_ptr(), segs, nseg, descs, n,
                                        int(bool(causal)), float(scale), o.data_ptr(), ls.data_ptr(),
                                        do.data_ptr(), workspace.data_ptr(), workspace.numel(), dq.data_ptr(),
                                        dk.data_ptr(), dv.data_ptr(), _stream(q))
    _check(lib, st, "ring_attention_backward")
    starts = [0]
    for ln in lens:
        starts.append(starts[-1] + ln)
    dks = [dk[:, :, a:a + ln] for a, ln in zip(starts, lens)]
    dvs = [dv[:, :, a:a + ln] for a, ln in zip(starts, lens)]
    return dq, dks, dvs
