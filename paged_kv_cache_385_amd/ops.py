"""Torch-facing wrappers of the C-ABI calls (marshalling only; every step runs in libpa).

Tensors must be contiguous, on one HIP device, in the dtypes and shapes pa.h
states.  Work is enqueued on the current torch stream unless ``stream`` is
given (a ``torch.cuda.Stream``).
"""

from __future__ import annotations

import ctypes as C
from typing import Optional, Tuple

import numpy as np
import torch

from . import _native as N

_DT = {torch.float16: N.PA_F16, torch.bfloat16: N.PA_BF16}


def k_pool_shape(num_blocks: int, num_kv_heads: int, head_dim: int) -> Tuple[int, ...]:
    return (num_blocks, num_kv_heads, head_dim // 8, N.BLOCK_SIZE, 8)


def v_pool_shape(num_blocks: int, num_kv_heads: int, head_dim: int) -> Tuple[int, ...]:
    return (num_blocks, num_kv_heads, N.BLOCK_SIZE // 4, head_dim, 4)


def k8_pool_shape(num_blocks: int, num_kv_heads: int, head_dim: int) -> Tuple[int, ...]:
    """FP8 K pool: [NB, Hkv, D/64, 16, 4, 2, 8] bytes (see pa.h)."""
    return (num_blocks, num_kv_heads, head_dim // 64, N.BLOCK_SIZE, 4, 2, 8)


def v8_pool_shape(num_blocks: int, num_kv_heads: int, head_dim: int) -> Tuple[int, ...]:
    """FP8 V pool: [NB, Hkv, 4, D/64, 16, 2, 2, 4] bytes (see pa.h)."""
    return (num_blocks, num_kv_heads, N.BLOCK_SIZE // 4, head_dim // 64, 16, 2, 2, 4)


def alloc_pool(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
               device="cuda", fill_bits: Optional[int] = None, fp8: bool = False
               ) -> Tuple[torch.Tensor, torch.Tensor]:
    """K and V pools in the library layout; ``fill_bits`` fills every element with a bit
    pattern (16-bit, or 8-bit for ``fp8`` pools, which are uint8 tensors of E4M3 codes)."""
    if fp8:
        k = torch.empty(k8_pool_shape(num_blocks, num_kv_heads, head_dim), dtype=torch.uint8, device=device)
        v = torch.empty(v8_pool_shape(num_blocks, num_kv_heads, head_dim), dtype=torch.uint8, device=device)
        if fill_bits is not None:
            k.fill_(int(fill_bits) & 0xFF)
            v.fill_(int(fill_bits) & 0xFF)
        return k, v
    k = torch.empty(k_pool_shape(num_blocks, num_kv_heads, head_dim), dtype=dtype, device=device)
    v = torch.empty(v_pool_shape(num_blocks, num_kv_heads, head_dim), dtype=dtype, device=device)
    if fill_bits is not None:
        val = int(np.int16(np.uint16(fill_bits)))
        k.view(torch.int16).fill_(val)
        v.view(torch.int16).fill_(val)
    return k, v


def _stream_ptr(stream, device) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return C.c_void_p(s.cuda_stream)


def cache_desc(k_cache: torch.Tensor, v_cache: torch.Tensor, shared_blocks: bool = False,
               scales: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
               dtype: Optional[torch.dtype] = None, host: bool = False) -> N.PaCache:
    """Descriptor of a pool pair; ``shared_blocks``: blocks may be shared within one call.

    FP8 pools (uint8 tensors of E4M3 codes) need ``scales`` = (k_scales, v_scales),
    float32 [Hkv] device tensors, and ``dtype``, the float16/bfloat16 dtype of q, out
    and of the k / v written into them.  ``host``: the pools are pinned host tensors
    (a swap tier), read and written by the device over the host link."""
    if host:
        if not (k_cache.is_pinned() and v_cache.is_pinned() and k_cache.is_contiguous()
                and v_cache.is_contiguous()):
            raise ValueError("host pools must be contiguous pinned tensors")
    elif not (k_cache.is_cuda and v_cache.is_cuda and k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("pools must be contiguous device tensors")
    shared = N.PA_CACHE_SHARED_BLOCKS if shared_blocks else 0
    if k_cache.dtype == torch.uint8:
        if v_cache.dtype != torch.uint8 or scales is None or dtype not in _DT:
            raise ValueError("FP8 pools need uint8 K and V, scales=(k_scales, v_scales) and dtype")
        nb, hkv, dp, bs = (int(x) for x in k_cache.shape[:4])
        D = dp * 64
        if (tuple(k_cache.shape) != k8_pool_shape(nb, hkv, D)
                or tuple(v_cache.shape) != v8_pool_shape(nb, hkv, D)):
            raise ValueError(f"FP8 pool shapes {tuple(k_cache.shape)} / {tuple(v_cache.shape)} "
                             "do not match the layout")
        ks, vs = scales
        for t, name in ((ks, "k_scales"), (vs, "v_scales")):
            _need(t, torch.float32, ks.device if host else k_cache.device, name, (hkv,))
        return N.PaCache(k_cache.data_ptr(), v_cache.data_ptr(), nb, bs, hkv, D, _DT[dtype],
                         shared | N.PA_CACHE_FP8, ks.data_ptr(), vs.data_ptr())
    if k_cache.dtype != v_cache.dtype or k_cache.dtype not in _DT:
        raise TypeError("pools must both be float16 or both bfloat16 (or uint8 FP8 codes)")
    nb, hkv, dc, bs, eight = k_cache.shape
    if eight != 8 or bs != N.BLOCK_SIZE or tuple(v_cache.shape) != v_pool_shape(nb, hkv, dc * 8):
        raise ValueError(f"pool shapes {tuple(k_cache.shape)} / {tuple(v_cache.shape)} do not match the layout")
    return N.PaCache(k_cache.data_ptr(), v_cache.data_ptr(), nb, bs, hkv, dc * 8, _DT[k_cache.dtype],
                     shared, None, None)


def _compute_dtype(k_cache: torch.Tensor, t: torch.Tensor) -> torch.dtype:
    """The float16/bfloat16 dtype of a call: the pool's, or (FP8 pools) the given tensor's."""
    return t.dtype if k_cache.dtype == torch.uint8 else k_cache.dtype


def _need(t: torch.Tensor, dtype, device, name, shape=None):
    if t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: need a contiguous {dtype} tensor on {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def cache_write(k_cache, v_cache, k, v, slot_mapping, stream=None, scales=None) -> None:
    dt = _compute_dtype(k_cache, k)
    desc = cache_desc(k_cache, v_cache, scales=scales, dtype=dt)
    T = k.shape[0]
    shp = (T, desc.num_kv_heads, desc.head_dim)
    _need(k, dt, k_cache.device, "k", shp)
    _need(v, dt, k_cache.device, "v", shp)
    _need(slot_mapping, torch.int64, k_cache.device, "slot_mapping", (T,))
    N.check(N.lib().pa_cache_write(C.byref(desc), k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                   T, _stream_ptr(stream, k_cache.device)), "pa_cache_write")


def copy_blocks(k_cache, v_cache, pairs, pairs_host: Optional[np.ndarray] = None, stream=None,
                scales=None) -> None:
    desc = cache_desc(k_cache, v_cache, scales=scales,
                      dtype=torch.bfloat16 if k_cache.dtype == torch.uint8 else None)
    n = pairs.shape[0]
    _need(pairs, torch.int32, k_cache.device, "pairs", (n, 2))
    host = None
    if pairs_host is not None:
        pairs_host = np.ascontiguousarray(pairs_host, dtype=np.int32)
        if pairs_host.shape != (n, 2):
            raise ValueError("pairs_host must match pairs")
        host = C.c_void_p(pairs_host.ctypes.data)
    N.check(N.lib().pa_copy_blocks(C.byref(desc), pairs.data_ptr(), host, n,
                                   _stream_ptr(stream, k_cache.device)), "pa_copy_blocks")


def swap_blocks(k_dev, v_dev, k_host, v_host, direction: int, pairs,
                pairs_host: Optional[np.ndarray] = None, stream=None, scales=None) -> None:
    """pa_swap_blocks: whole-block copies between device pools and pinned host pools of the
    same layout; ``direction`` N.PA_SWAP_OUT (pairs (device, host)) or N.PA_SWAP_IN
    (pairs (host, device)); ``pairs`` int32 [n, 2] on the device."""
    dt = torch.bfloat16 if k_dev.dtype == torch.uint8 else None
    dd = cache_desc(k_dev, v_dev, scales=scales, dtype=dt)
    hd = cache_desc(k_host, v_host, scales=scales, dtype=dt, host=True)
    n = pairs.shape[0]
    _need(pairs, torch.int32, k_dev.device, "pairs", (n, 2))
    host = None
    if pairs_host is not None:
        pairs_host = np.ascontiguousarray(pairs_host, dtype=np.int32)
        if pairs_host.shape != (n, 2):
            raise ValueError("pairs_host must match pairs")
        host = C.c_void_p(pairs_host.ctypes.data)
    N.check(N.lib().pa_swap_blocks(C.byref(dd), C.byref(hd), direction, pairs.data_ptr(), host, n,
                                   _stream_ptr(stream, k_dev.device)), "pa_swap_blocks")


def workspace_size(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int) -> int:
    return int(N.lib().pa_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len))


def alloc_workspace(num_seqs, num_heads, head_dim, max_context_len, device="cuda") -> torch.Tensor:
    """Zero-filled workspace: its leading counters must be zero before the first call."""
    n = workspace_size(num_seqs, num_heads, head_dim, max_context_len)
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def workspace_counter_bytes(num_seqs: int, num_heads: int) -> int:
    """Bytes of the workspace's leading counter region (kept zero between calls): the
    merge counters int32[B][H] and one claim counter."""
    return (4 * (num_seqs * num_heads + 1) + 255) // 256 * 256


def _decode_args(k_cache, v_cache, q, block_tables, context_lens, out, workspace,
                 shared_blocks=False, scales=None):
    dt = _compute_dtype(k_cache, q)
    desc = cache_desc(k_cache, v_cache, shared_blocks, scales=scales, dtype=dt)
    B, H, D = q.shape
    _need(q, dt, k_cache.device, "q")
    if D != desc.head_dim:
        raise ValueError("q head_dim differs from the pool's")
    _need(block_tables, torch.int32, k_cache.device, "block_tables")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    _need(context_lens, torch.int32, k_cache.device, "context_lens", (B,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, dt, k_cache.device, "out", (B, H, D))
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    return desc, B, H, out, ws_ptr, ws_bytes


def decode(k_cache, v_cache, q, block_tables, context_lens, max_context_len: int, scale: float,
           out=None, workspace=None, stream=None, shared_blocks: bool = False,
           scales=None) -> torch.Tensor:
    """pa_decode: attention pass then log-sum-exp merge; returns out [B, H, D]."""
    desc, B, H, out, ws, wsb = _decode_args(k_cache, v_cache, q, block_tables, context_lens, out,
                                            workspace, shared_blocks, scales)
    N.check(N.lib().pa_decode(C.byref(desc), q.data_ptr(), B, H, block_tables.data_ptr(),
                              block_tables.shape[1], context_lens.data_ptr(), max_context_len,
                              scale, out.data_ptr(), ws, wsb, _stream_ptr(stream, q.device)),
            "pa_decode")
    return out


def decode_noalloc(k_cache, v_cache, q, block_tables, context_lens, max_context_len: int,
                   scale: float, out=None, stream=None, scales=None) -> torch.Tensor:
    """pa_decode_noalloc: pa_decode on the library's own scratch (no workspace); returns
    out [B, H, D].  Calls that may overlap on one device race on that scratch."""
    desc, B, H, out, _, _ = _decode_args(k_cache, v_cache, q, block_tables, context_lens, out,
                                         None, False, scales)
    N.check(N.lib().pa_decode_noalloc(C.byref(desc), q.data_ptr(), B, H, block_tables.data_ptr(),
                                      block_tables.shape[1], context_lens.data_ptr(),
                                      max_context_len, scale, out.data_ptr(),
                                      _stream_ptr(stream, q.device)), "pa_decode_noalloc")
    return out


def decode_partitioned(k_cache, v_cache, q, block_tables, context_lens, max_context_len: int,
                       scale: float, partition_tokens: int, out=None, workspace=None, stream=None,
                       scales=None) -> torch.Tensor:
    """pa_decode_partitioned: pa_decode with a fixed partition length (512 .. 4096 tokens,
    or 0 for the per-launch choice); returns out [B, H, D]."""
    desc, B, H, out, ws, wsb = _decode_args(k_cache, v_cache, q, block_tables, context_lens, out,
                                            workspace, False, scales)
    N.check(N.lib().pa_decode_partitioned(C.byref(desc), q.data_ptr(), B, H,
                                          block_tables.data_ptr(), block_tables.shape[1],
                                          context_lens.data_ptr(), max_context_len, scale,
                                          int(partition_tokens), out.data_ptr(), ws, wsb,
                                          _stream_ptr(stream, q.device)), "pa_decode_partitioned")
    return out


def group_plan(tables: np.ndarray, context_lens: np.ndarray, max_context_len: int, num_heads: int,
               num_kv_heads: int, min_items: int = 1024) -> np.ndarray:
    """pa_group_plan on host arrays: the grouped-decode plan (int32), empty when grouping
    the batch by shared prefix would not pay."""
    tab = np.ascontiguousarray(tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, mb = tab.shape
    nbytes = int(N.lib().pa_group_plan_bytes(B, max_context_len))
    plan = np.zeros(max(nbytes // 4, 1), dtype=np.int32)
    n = C.c_int32()
    N.check(N.lib().pa_group_plan(tab.ctypes.data, B, mb, ctx.ctypes.data, max_context_len,
                                  num_heads, num_kv_heads, min_items, plan.ctypes.data, nbytes,
                                  C.byref(n)), "pa_group_plan")
    return plan[:n.value].copy()


def decode_grouped(k_cache, v_cache, q, block_tables, max_context_len: int, scale: float,
                   plan: np.ndarray, out=None, workspace=None, stream=None, scales=None,
                   shared_blocks: bool = True) -> torch.Tensor:
    """pa_decode_grouped with a plan from ``group_plan`` (uploaded here); returns out."""
    dt = _compute_dtype(k_cache, q)
    desc = cache_desc(k_cache, v_cache, shared_blocks, scales=scales, dtype=dt)
    B, H, D = q.shape
    _need(q, dt, k_cache.device, "q")
    _need(block_tables, torch.int32, k_cache.device, "block_tables")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, dt, k_cache.device, "out", (B, H, D))
    plan_h = np.ascontiguousarray(plan, dtype=np.int32)
    plan_d = torch.from_numpy(plan_h).to(k_cache.device)
    ws, wsb = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                   workspace.numel() * workspace.element_size())
    N.check(N.lib().pa_decode_grouped(C.byref(desc), q.data_ptr(), B, H, block_tables.data_ptr(),
                                      block_tables.shape[1], max_context_len, plan_d.data_ptr(),
                                      plan_h.ctypes.data, scale, out.data_ptr(), ws, wsb,
                                      _stream_ptr(stream, q.device)), "pa_decode_grouped")
    return out


def decode_fused(k_cache, v_cache, k_new, v_new, slot_mapping, q, block_tables, context_lens,
                 max_context_len: int, scale: float, out=None, workspace=None,
                 stream=None, scales=None) -> torch.Tensor:
    """pa_decode_fused: store each sequence's newest token, then decode; returns out [B, H, D]."""
    desc, B, H, out, ws, wsb = _decode_args(k_cache, v_cache, q, block_tables, context_lens, out,
                                            workspace, False, scales)
    shp = (B, desc.num_kv_heads, desc.head_dim)
    _need(k_new, q.dtype, k_cache.device, "k_new", shp)
    _need(v_new, q.dtype, k_cache.device, "v_new", shp)
    _need(slot_mapping, torch.int64, k_cache.device, "slot_mapping", (B,))
    N.check(N.lib().pa_decode_fused(C.byref(desc), k_new.data_ptr(), v_new.data_ptr(),
                                    slot_mapping.data_ptr(), q.data_ptr(), B, H,
                                    block_tables.data_ptr(), block_tables.shape[1],
                                    context_lens.data_ptr(), max_context_len, scale, out.data_ptr(),
                                    ws, wsb, _stream_ptr(stream, q.device)), "pa_decode_fused")
    return out


def decode_attention(k_cache, v_cache, q, block_tables, context_lens, max_context_len: int,
                     scale: float, out=None, workspace=None, stream=None,
                     scales=None) -> torch.Tensor:
    desc, B, H, out, ws, wsb = _decode_args(k_cache, v_cache, q, block_tables, context_lens, out,
                                            workspace, False, scales)
    N.check(N.lib().pa_decode_attention(C.byref(desc), q.data_ptr(), B, H, block_tables.data_ptr(),
                                        block_tables.shape[1], context_lens.data_ptr(),
                                        max_context_len, scale, out.data_ptr(), ws, wsb,
                                        _stream_ptr(stream, q.device)), "pa_decode_attention")
    return out


def decode_merge(k_cache, v_cache, context_lens, max_context_len: int, out, workspace=None,
                 stream=None, scales=None) -> torch.Tensor:
    desc = cache_desc(k_cache, v_cache, scales=scales, dtype=_compute_dtype(k_cache, out))
    B, H, D = out.shape
    _need(context_lens, torch.int32, k_cache.device, "context_lens", (B,))
    ws, wsb = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                   workspace.numel() * workspace.element_size())
    N.check(N.lib().pa_decode_merge(C.byref(desc), B, H, context_lens.data_ptr(), max_context_len,
                                    out.data_ptr(), ws, wsb, _stream_ptr(stream, out.device)),
            "pa_decode_merge")
    return out


def chunk_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                         total_q: int, max_q_len: int, max_context_len: int) -> int:
    return int(N.lib().pa_chunk_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, total_q,
                                               max_q_len, max_context_len))


def chunk_attention(k_cache, v_cache, q, q_starts, block_tables, context_lens, max_q_len: int,
                    max_context_len: int, scale: float, out=None, workspace=None,
                    stream=None, scales=None, events=None) -> torch.Tensor:
    """pa_chunk_attention: the last q_len_b tokens of each sequence (rows q_starts[b] ..
    q_starts[b+1] of the packed q [total, H, D]) attend causally over its cache.
    Returns out [total, H, D]; allocates the workspace when none is given.  FP8 pools
    take ``scales`` = (k_scales, v_scales); q and out are then float16 or bfloat16.
    ``events`` (optional): a (begin, end) pair of torch.cuda.Event, already recorded
    once, attached to the kernels' dispatches (start of attention, end of the call)."""
    dt = _compute_dtype(k_cache, q)
    desc = cache_desc(k_cache, v_cache, scales=scales, dtype=dt)
    dev = k_cache.device
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError(f"q must be [total, H, {desc.head_dim}], got {tuple(q.shape)}")
    T, H = int(q.shape[0]), int(q.shape[1])
    B = int(q_starts.shape[0]) - 1
    _need(q, dt, dev, "q")
    _need(q_starts, torch.int32, dev, "q_starts", (B + 1,))
    _need(block_tables, torch.int32, dev, "block_tables")
    _need(context_lens, torch.int32, dev, "context_lens", (B,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, dt, dev, "out", tuple(q.shape))
    need = chunk_workspace_size(B, H, desc.num_kv_heads, desc.head_dim, T, max_q_len,
                                max_context_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws = workspace.data_ptr() if workspace is not None else None
    wsb = workspace.numel() if workspace is not None else 0
    N.check(N.lib().pa_chunk_attention(C.byref(desc), q.data_ptr(), q_starts.data_ptr(), B, T,
                                       max_q_len, H, block_tables.data_ptr(), block_tables.shape[1],
                                       context_lens.data_ptr(), max_context_len, scale,
                                       out.data_ptr(), ws, wsb,
                                       events[0].cuda_event if events else None,
                                       events[1].cuda_event if events else None,
                                       _stream_ptr(stream, dev)),
            "pa_chunk_attention")
    return out
