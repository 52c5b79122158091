"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The compute runs in libpa.so (hand-written HIP kernels plus a C++ host block
manager, C ABI in include/pa.h); this package only marshals arguments.
"""

from . import _native  # noqa: F401
from .block_manager import BlockManager  # noqa: F401
from .ops import (alloc_pool, alloc_workspace, cache_desc, cache_write, chunk_attention,  # noqa: F401
                  chunk_workspace_size, copy_blocks, decode, decode_attention, decode_fused,
                  decode_grouped, decode_merge, decode_noalloc, decode_partitioned,
                  group_plan, workspace_size)
from .engine import DecodeBatch, PagedKVCache  # noqa: F401

__all__ = ["BlockManager", "PagedKVCache", "DecodeBatch", "alloc_pool", "alloc_workspace",
           "cache_desc", "cache_write", "chunk_attention", "chunk_workspace_size", "copy_blocks",
           "decode", "decode_attention", "decode_fused", "decode_grouped", "decode_merge",
           "decode_noalloc", "decode_partitioned", "group_plan", "workspace_size"]
