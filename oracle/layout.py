"""Physical block layout of the HIP library's pools.  TEST INFRASTRUCTURE ONLY.

The pages leave the in-memory layout of a block open ("vLLM 核心概念", section
"核心概念：块（Block）" only says a block holds the K and V of 16 tokens).  The
library's layout is its own design, documented in its C header; this module
restates that documentation as a view onto the logical pool
``[num_blocks, num_kv_heads, block_size, head_dim]`` so tests can compare a
device pool with the oracle's.  It is an encoding, pinned by the hand-worked
offsets in ``tests/golden/layout_offsets.json``.

K pool, physical shape ``[NB, Hkv, D/8, bs, 8]``:
    element (block b, head h, token t, dim d) sits at [b, h, d // 8, t, d % 8].
V pool, physical shape ``[NB, Hkv, bs/4, D, 4]``:
    element (block b, head h, token t, dim d) sits at [b, h, t // 4, d, t % 4].
"""

from __future__ import annotations

import numpy as np


def k_physical_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 16):
    return (num_blocks, num_kv_heads, head_dim // 8, block_size, 8)


def v_physical_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 16):
    return (num_blocks, num_kv_heads, block_size // 4, head_dim, 4)


def k_to_logical(kphys: np.ndarray) -> np.ndarray:
    nb, hkv, dc, bs, eight = kphys.shape
    return kphys.transpose(0, 1, 3, 2, 4).reshape(nb, hkv, bs, dc * eight)


def v_to_logical(vphys: np.ndarray) -> np.ndarray:
    nb, hkv, tq, d, four = vphys.shape
    return vphys.transpose(0, 1, 2, 4, 3).reshape(nb, hkv, tq * four, d)


def k_from_logical(klog: np.ndarray) -> np.ndarray:
    nb, hkv, bs, d = klog.shape
    return np.ascontiguousarray(klog.reshape(nb, hkv, bs, d // 8, 8).transpose(0, 1, 3, 2, 4))


def v_from_logical(vlog: np.ndarray) -> np.ndarray:
    nb, hkv, bs, d = vlog.shape
    return np.ascontiguousarray(vlog.reshape(nb, hkv, bs // 4, 4, d).transpose(0, 1, 2, 4, 3))


# ---- FP8 (E4M3 codes, one byte per element) pools --------------------------------
# One (block, head) tile is 16 * D bytes.  K, physical [NB, Hkv, D/64, bs, 4, 2, 8]:
#     element (b, h, t, d) sits at [b, h, d // 64, t, (d % 32) // 8, (d % 64) // 32, d % 8],
# so 16 consecutive bytes hold dims 8g .. 8g+7 and 32+8g .. 32+8g+7 (of one 64-dim
# group) of one token.  V, physical [NB, Hkv, bs/4, D/64, 16, 2, 2, 4] -- read as
# [b, h, t // 4, d // 64, (d % 32) // 2, (d % 64) // 32, d % 2, t % 4]:
# 16 consecutive bytes hold dims (2n, 2n+1) and (32+2n, 33+2n) of 4 tokens.


def k8_physical_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 16):
    return (num_blocks, num_kv_heads, head_dim // 64, block_size, 4, 2, 8)


def v8_physical_shape(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 16):
    return (num_blocks, num_kv_heads, block_size // 4, head_dim // 64, 16, 2, 2, 4)


def k8_to_logical(kphys: np.ndarray) -> np.ndarray:
    nb, hkv, dp, bs, g4, kk, e = kphys.shape
    # [b, h, p, t, g4, kk, e] -> [b, h, t, p, kk, g4, e]; d = 64 p + 32 kk + 8 g4 + e
    return kphys.transpose(0, 1, 3, 2, 5, 4, 6).reshape(nb, hkv, bs, dp * kk * g4 * e)


def k8_from_logical(klog: np.ndarray) -> np.ndarray:
    nb, hkv, bs, d = klog.shape
    x = klog.reshape(nb, hkv, bs, d // 64, 2, 4, 8)          # [b, h, t, p, kk, g4, e]
    return np.ascontiguousarray(x.transpose(0, 1, 3, 2, 5, 4, 6))


def v8_to_logical(vphys: np.ndarray) -> np.ndarray:
    nb, hkv, tq, dq, n, j2, dd, tt = vphys.shape
    # [b, h, tq, q, n, j2, dd, tt] -> [b, h, tq, tt, q, j2, n, dd]; t = 4 tq + tt,
    # d = 64 q + 32 j2 + 2 n + dd
    x = vphys.transpose(0, 1, 2, 7, 3, 5, 4, 6)
    return x.reshape(nb, hkv, tq * tt, dq * j2 * n * dd)


def v8_from_logical(vlog: np.ndarray) -> np.ndarray:
    nb, hkv, bs, d = vlog.shape
    x = vlog.reshape(nb, hkv, bs // 4, 4, d // 64, 2, 16, 2)  # [b, h, tq, tt, q, j2, n, dd]
    return np.ascontiguousarray(x.transpose(0, 1, 2, 4, 6, 5, 7, 3))
