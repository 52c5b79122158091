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
