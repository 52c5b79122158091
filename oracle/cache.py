"""Slot-mapped cache write, block copy and block-table gather.  TEST INFRASTRUCTURE ONLY.

The logical pool is a pair of arrays K, V of shape
``[num_blocks, num_kv_heads, block_size, head_dim]`` holding 16-bit patterns
(uint16), so every copy is bit-exact whatever the float dtype.

* A block stores the K and V vectors of a fixed number of tokens, 16 by
  default ("vLLM 核心概念", section "核心概念：块（Block）").
* A sequence's logical blocks map to physical blocks through its block table;
  tokens 0-15 live in the block of entry 0, 16-31 in entry 1, and so on
  (same page, section "逻辑视图与物理视图分离").
* Slot encoding (the pages are silent; reading): a token's slot is
  ``physical_block * block_size + position_in_block``; a negative slot means
  "do not store this token".
* The current token's K and V are stored before attention reuses them
  ("vLLM 核心概念", section "为什么需要 KV Cache？").
* Copy-on-write copies a whole block, K and V, from a shared source to a
  fresh destination ("理解 vLLM PagedAttention", section 六).
"""

from __future__ import annotations

import numpy as np


def bits16(x) -> np.ndarray:
    """uint16 bit patterns of a 16-bit float array or CPU torch tensor."""
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return x
    if x.dtype == np.float16:
        return x.view(np.uint16)
    raise TypeError(f"not a 16-bit array: {x.dtype}")


def empty_pool(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 16,
               fill: int = 0) -> tuple[np.ndarray, np.ndarray]:
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    return (np.full(shape, fill, dtype=np.uint16), np.full(shape, fill, dtype=np.uint16))


def cache_write(kpool: np.ndarray, vpool: np.ndarray, k, v, slots, inplace: bool = False
                ) -> tuple[np.ndarray, np.ndarray]:
    """Pools with token t's K/V [Hkv, D] stored at slot ``slots[t]`` (copies unless ``inplace``)."""
    if not inplace:
        kpool = kpool.copy()
        vpool = vpool.copy()
    kb, vb = bits16(k), bits16(v)
    bs = kpool.shape[2]
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        kpool[blk, :, off, :] = kb[t]
        vpool[blk, :, off, :] = vb[t]
    return kpool, vpool


def copy_blocks(kpool: np.ndarray, vpool: np.ndarray, pairs, inplace: bool = False
                ) -> tuple[np.ndarray, np.ndarray]:
    """Pools with block dst := block src for every (src, dst) pair (copies unless ``inplace``).

    Pairs are applied one after another.  When destinations are distinct and
    none is also a source (what a copy-on-write list always satisfies), the
    order does not matter.
    """
    if not inplace:
        kpool = kpool.copy()
        vpool = vpool.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        kpool[dst] = kpool[src]
        vpool[dst] = vpool[src]
    return kpool, vpool


def gather_sequence(kpool: np.ndarray, vpool: np.ndarray, table, ctx: int
                    ) -> tuple[np.ndarray, np.ndarray]:
    """Contiguous [ctx, Hkv, D] K and V of a sequence, read through its block table."""
    bs = kpool.shape[2]
    idx_blk = np.array([table[t // bs] for t in range(ctx)], dtype=np.int64)
    idx_off = np.array([t % bs for t in range(ctx)], dtype=np.int64)
    return kpool[idx_blk, :, idx_off, :], vpool[idx_blk, :, idx_off, :]


def scatter_sequence(kpool: np.ndarray, vpool: np.ndarray, table, k, v
                     ) -> tuple[np.ndarray, np.ndarray]:
    """Place a contiguous sequence [ctx, Hkv, D] into the blocks its table names."""
    bs = kpool.shape[2]
    ctx = k.shape[0]
    slots = [int(table[t // bs]) * bs + t % bs for t in range(ctx)]
    return cache_write(kpool, vpool, k, v, slots)


# ---- FP8 pools: E4M3 codes, one float32 scale per KV head for K and one for V --------
def empty_pool8(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 16,
                fill: int = 0) -> tuple[np.ndarray, np.ndarray]:
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    return (np.full(shape, fill, dtype=np.uint8), np.full(shape, fill, dtype=np.uint8))


def cache_write8(kpool: np.ndarray, vpool: np.ndarray, k, v, slots, k_scales, v_scales,
                 inplace: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """FP8 pools with token t's K/V [Hkv, D] quantised (per KV head h: encode(fp32(x) /
    fp32(scale_h))) at slot ``slots[t]``; copies unless ``inplace``."""
    from oracle import fp8
    if not inplace:
        kpool = kpool.copy()
        vpool = vpool.copy()
    kf = k.detach().to("cpu").float().numpy() if hasattr(k, "detach") else np.asarray(k, np.float32)
    vf = v.detach().to("cpu").float().numpy() if hasattr(v, "detach") else np.asarray(v, np.float32)
    ks = np.asarray(k_scales, dtype=np.float32)[:, None]
    vs = np.asarray(v_scales, dtype=np.float32)[:, None]
    bs = kpool.shape[2]
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        kpool[blk, :, off, :] = fp8.quantize(kf[t], ks)
        vpool[blk, :, off, :] = fp8.quantize(vf[t], vs)
    return kpool, vpool


def dequant_sequence8(kpool: np.ndarray, vpool: np.ndarray, table, ctx: int, k_scales, v_scales
                      ) -> tuple[np.ndarray, np.ndarray]:
    """float64 [ctx, Hkv, D] K and V values of a sequence in FP8 pools (code * scale)."""
    from oracle import fp8
    kc, vc = gather_sequence(kpool, vpool, table, ctx)
    ks = np.asarray(k_scales, dtype=np.float32)[None, :, None]
    vs = np.asarray(v_scales, dtype=np.float32)[None, :, None]
    return fp8.dequantize(kc, ks), fp8.dequantize(vc, vs)
