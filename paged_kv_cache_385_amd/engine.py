"""One GPU's paged KV cache and the decode step that drives it.

``PagedKVCache`` owns a K/V pool pair in the library layout and a native
block manager.  ``DecodeBatch`` runs decode steps for a fixed set of
sequences; one step is the whole hot path, in this order:

1. host: the block manager reserves each sequence's next slot (and reports
   copy-on-write pairs), then packs block tables and context lengths;
2. one pinned host-to-device copy of slots, lengths, tables and pairs;
3. ``pa_copy_blocks`` for the pairs (before any write can land in a block
   that is still shared);
4. ``pa_cache_write`` of the new tokens' K and V;
5. ``pa_decode_attention`` then ``pa_decode_merge``.

The copy-before-write order follows copy-on-write as "理解 vLLM PagedAttention"
section 六 describes it: a diverging sequence must get its private copy of
the shared block before its new token is stored.
"""

from __future__ import annotations

from typing import Callable, Iterable, Optional, Sequence, Tuple

import numpy as np
import torch

from . import _native as N
from . import ops
from .block_manager import BlockManager

_ALIGN = 256


class PagedKVCache:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
                 device="cuda", free_order: Optional[Sequence[int]] = None,
                 fill_bits: Optional[int] = None):
        self.num_blocks = num_blocks
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.dtype = dtype
        self.device = torch.device(device)
        self.k_cache, self.v_cache = ops.alloc_pool(num_blocks, num_kv_heads, head_dim, dtype,
                                                    self.device, fill_bits)
        self.bm = BlockManager(num_blocks, N.BLOCK_SIZE, free_order)

    # ---- device operations ----------------------------------------------------------
    def write(self, k: torch.Tensor, v: torch.Tensor, slots) -> None:
        if isinstance(slots, np.ndarray):
            slots = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).to(self.device)
        ops.cache_write(self.k_cache, self.v_cache, k.to(self.device), v.to(self.device), slots)

    def copy(self, pairs: np.ndarray) -> None:
        pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
        if len(pairs) == 0:
            return
        ops.copy_blocks(self.k_cache, self.v_cache, torch.from_numpy(pairs).to(self.device),
                        pairs_host=pairs)

    # ---- trace replay ----------------------------------------------------------------
    def apply_trace(self, trace: Iterable[tuple],
                    token_kv: Callable[[int, int, int], Tuple[torch.Tensor, torch.Tensor]],
                    on_cow: Optional[Callable[[np.ndarray], None]] = None) -> None:
        """Replay block-manager operations and their device work, one operation at a time.

        trace entries: ("add", sid) | ("fork", parent, child) |
        ("append", sid, seg, start, n) whose K/V are ``token_kv(seg, start, n)``.
        Each append copies the blocks it had to copy before it writes: the
        last sharer of a block only writes in place after every other sharer
        has taken its copy, so operation order keeps every copy valid.
        """
        for op in trace:
            if op[0] == "add":
                self.bm.add_seq(op[1])
            elif op[0] == "fork":
                self.bm.fork(op[1], op[2])
            elif op[0] == "append":
                _, sid, seg, start, n = op
                slots, cows = self.bm.append_tokens(sid, n)
                if len(cows):
                    self.copy(cows)
                    if on_cow is not None:
                        on_cow(cows)
                k, v = token_kv(seg, start, n)
                self.write(k, v, slots)
            else:
                raise ValueError(f"unknown operation {op[0]}")

    def tables(self, sids: Sequence[int], max_blocks: int) -> Tuple[torch.Tensor, torch.Tensor, int]:
        """Device block tables and context lengths for ``sids``, plus the host max context."""
        tab, ctx = self.bm.pack(sids, max_blocks)
        return (torch.from_numpy(tab).to(self.device), torch.from_numpy(ctx).to(self.device),
                int(ctx.max()) if len(ctx) else 1)


class DecodeBatch:
    """Decode steps for a fixed list of sequences on one stream (see module docstring)."""

    def __init__(self, cache: PagedKVCache, sids: Sequence[int], num_heads: int, scale: float,
                 max_blocks_per_seq: int, stream: Optional[torch.cuda.Stream] = None):
        self.cache = cache
        self.sids = np.ascontiguousarray(np.asarray(sids, dtype=np.int64))
        self.B = B = len(self.sids)
        self.H = num_heads
        self.scale = float(scale)
        self.max_blocks = max_blocks_per_seq
        self.stream = stream if stream is not None else torch.cuda.current_stream(cache.device)
        dev = cache.device
        # one staging region: slots int64[B] | ctx int32[B] | tables int32[B*MB] | pairs int32[B*2]
        self._off = []
        off = 0
        for nbytes in (8 * B, 4 * B, 4 * B * max_blocks_per_seq, 8 * B):
            self._off.append(off)
            off += (nbytes + _ALIGN - 1) // _ALIGN * _ALIGN
        self._bytes = off
        self._pinned = [torch.empty(off, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        self._staged = [torch.cuda.Event() for _ in range(2)]
        self._dev = torch.empty(off, dtype=torch.uint8, device=dev)
        self.slots_d = self._view(self._dev, 0, torch.int64, (B,))
        self.ctx_d = self._view(self._dev, 1, torch.int32, (B,))
        self.tables_d = self._view(self._dev, 2, torch.int32, (B, max_blocks_per_seq))
        self.pairs_d = self._view(self._dev, 3, torch.int32, (B, 2))
        self.out = torch.empty((B, num_heads, cache.head_dim), dtype=cache.dtype, device=dev)
        self.workspace = ops.alloc_workspace(B, num_heads, cache.head_dim,
                                             max_blocks_per_seq * N.BLOCK_SIZE, dev)
        self._i = 0
        self.last_max_ctx = 0
        self.last_pairs = np.zeros((0, 2), dtype=np.int32)

    def _view(self, buf: torch.Tensor, i: int, dtype, shape):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        return buf[self._off[i]:self._off[i] + n].view(dtype).view(*shape)

    def reserve(self) -> int:
        """Host part of a step: reserve slots, pack tables, stage and upload.  Returns max context."""
        buf = self._i & 1
        self._i += 1
        self._staged[buf].synchronize()          # the copy that last read this buffer is done
        pin = self._pinned[buf]
        slots = self._view(pin, 0, torch.int64, (self.B,)).numpy()
        ctx = self._view(pin, 1, torch.int32, (self.B,)).numpy()
        tabs = self._view(pin, 2, torch.int32, (self.B, self.max_blocks)).numpy()
        pairs = self._view(pin, 3, torch.int32, (self.B, 2)).numpy()
        _, cows = self.cache.bm.append_batch(self.sids, slots_out=slots)
        pairs[:len(cows)] = cows
        self.cache.bm.pack(self.sids, self.max_blocks, tables_out=tabs, ctx_out=ctx)
        with torch.cuda.stream(self.stream):
            self._dev.copy_(pin, non_blocking=True)
            self._staged[buf].record(self.stream)
        self.last_pairs = cows.copy()
        self.last_max_ctx = int(ctx.max())
        return self.last_max_ctx

    def step(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
             attn_events: Optional[Tuple[torch.cuda.Event, torch.cuda.Event]] = None) -> torch.Tensor:
        """One decode step (host reservation included).  Returns the output tensor (reused)."""
        max_ctx = self.reserve()
        c = self.cache
        n_cow = len(self.last_pairs)
        s = self.stream
        if n_cow:
            ops.copy_blocks(c.k_cache, c.v_cache, self.pairs_d[:n_cow], pairs_host=self.last_pairs,
                            stream=s)
        ops.cache_write(c.k_cache, c.v_cache, k_new, v_new, self.slots_d, stream=s)
        if attn_events is not None:
            attn_events[0].record(s)
        ops.decode_attention(c.k_cache, c.v_cache, q, self.tables_d, self.ctx_d, max_ctx, self.scale,
                             out=self.out, workspace=self.workspace, stream=s)
        if attn_events is not None:
            attn_events[1].record(s)
        ops.decode_merge(c.k_cache, c.v_cache, self.ctx_d, max_ctx, self.out,
                         workspace=self.workspace, stream=s)
        return self.out
