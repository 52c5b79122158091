"""One GPU's paged KV cache and the decode step that drives it.

``PagedKVCache`` owns a K/V pool pair in the library layout and a native
block manager.  ``DecodeBatch`` runs decode steps for a fixed set of
sequences; one step is the whole hot path, done by one native call
(``pa_decode_step``), in this order:

1. host: the block manager reserves each sequence's next slot (and reports
   copy-on-write pairs), then packs block tables and context lengths into a
   pinned staging buffer;
2. one host-to-device copy of that buffer (none for a tiny batch, whose kernels
   read it in place);
3. ``pa_copy_blocks`` for the pairs (before any write can land in a block
   that is still shared);
4. ``pa_cache_write`` of the new tokens' K and V;
5. the attention pass then the log-sum-exp merge.

The copy-before-write order follows copy-on-write as "理解 vLLM PagedAttention"
section 六 describes it: a diverging sequence must get its private copy of
the shared block before its new token is stored.
"""

from __future__ import annotations

import ctypes as C
from typing import Callable, Iterable, Optional, Sequence, Tuple

import numpy as np
import torch

from . import _native as N
from . import ops
from .block_manager import BlockManager

_ALIGN = 256
# Default staging of a DecodeBatch: batches whose K/V can never exceed this many bytes
# decode in tens of microseconds, and their kernels reading the staged tables in place
# ("mapped") beat a copy plus its wait; larger batches copy on a side stream ("side").
_MAPPED_MAX_KV_BYTES = 16 << 20
# Staging slots of a DecodeBatch: up to this many, holding together at most this many
# pinned bytes.  An event recorded on a stream between two kernels delays the second
# by about 5.5 us on gfx950, so the step marks its completion only once per half ring.
_RING_MAX = 16
_RING_BYTES = 32 << 20


def _round(n: int) -> int:
    return (n + _ALIGN - 1) // _ALIGN * _ALIGN


def _ring_slots(staging_bytes: int) -> int:
    """Staging slots for one step's ``staging_bytes``: even, 2 .. _RING_MAX."""
    return max(2, min(_RING_MAX, _RING_BYTES // max(1, staging_bytes)) & ~1)


class _CompletionMarks:
    """Which kernels of a step ring have finished, from one event per ``every`` steps.

    Step i records a mark after its kernels when i % every == every - 1 (``after``).
    ``wait(j)`` returns once the kernels of step j (and of every step before it on the
    stream) have finished: it waits for the first mark at or after step j, which a
    ring of 2 * every slots always holds before the slot of step j is reused, and
    recycles the older marks' events.  A step whose call failed records no mark; when
    no mark is in range, ``wait`` drains the stream instead (``drain``).  ``new_event``
    makes an event, ``record`` records one on the stream, ``sync`` waits for one (host
    side); all are plain callables so the bookkeeping runs without a device.
    """

    def __init__(self, every: int, new_event: Callable, record: Callable, sync: Callable,
                 drain: Callable):
        self.every = every
        self._new, self._record, self._sync, self._drain = new_event, record, sync, drain
        self._marks = []          # (step, event), oldest first
        self._spare = []

    def prime(self, n: int) -> None:
        """Make and record ``n`` spare events now (an event's first record creates it)."""
        for _ in range(n):
            ev = self._new()
            self._record(ev)
            self._spare.append(ev)

    def after(self, i: int) -> None:
        if i % self.every == self.every - 1:
            ev = self._spare.pop() if self._spare else self._new()
            self._record(ev)
            self._marks.append((i, ev))

    def wait(self, j: int) -> None:
        if j < 0:
            return
        k = 0
        while k < len(self._marks) and self._marks[k][0] < j:
            k += 1
        self._spare.extend(ev for _, ev in self._marks[:k])
        if k == len(self._marks):
            del self._marks[:]
            self._drain()
            return
        del self._marks[:k]
        self._sync(self._marks[0][1])


class PagedKVCache:
    """K/V pools, their host block manager, and the device operations on them.

    ``dtype`` is the float16/bfloat16 dtype of the tokens written and of q/out.  With
    ``kv_scales`` = (k_scales, v_scales) -- one positive float per KV head each -- the
    pools hold 8-bit E4M3 codes of x / scale instead (``PA_CACHE_FP8``).  With
    ``prefix_caching`` the block manager indexes committed full blocks and ``admit``
    reuses them for requests whose prompts share a prefix.  With ``host_blocks`` > 0 a
    host tier of that many blocks (pinned host pools of the same layout) takes
    swapped-out sequences (``swap_out`` / ``swap_in``)."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
                 device="cuda", free_order: Optional[Sequence[int]] = None,
                 fill_bits: Optional[int] = None, kv_scales=None, prefix_caching: bool = False,
                 host_blocks: int = 0, block_size: int = N.BLOCK_SIZE):
        self.num_blocks = num_blocks
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.dtype = dtype
        self.device = torch.device(device)
        self.fp8 = kv_scales is not None
        self.scales = None
        if self.fp8:
            self.scales = tuple(torch.as_tensor(np.asarray(s, dtype=np.float32)).reshape(num_kv_heads)
                                .to(self.device).contiguous() for s in kv_scales)
        self.k_cache, self.v_cache = ops.alloc_pool(num_blocks, num_kv_heads, head_dim, dtype,
                                                    self.device, fill_bits, fp8=self.fp8)
        # a 32-token manager block is two adjacent 16-token tiles of the pool
        self.tiles_per_block = block_size // N.BLOCK_SIZE
        if block_size not in (16, 32) or num_blocks % self.tiles_per_block:
            raise ValueError("block_size must be 16 or 32, dividing num_blocks into tile pairs")
        self.bm = BlockManager(num_blocks // self.tiles_per_block, block_size, free_order,
                               prefix_caching)
        self.k_host = self.v_host = None
        if host_blocks > 0:
            shp = (ops.k8_pool_shape if self.fp8 else ops.k_pool_shape)(host_blocks, num_kv_heads, head_dim)
            vshp = (ops.v8_pool_shape if self.fp8 else ops.v_pool_shape)(host_blocks, num_kv_heads, head_dim)
            pdt = torch.uint8 if self.fp8 else dtype
            self.k_host = torch.zeros(shp, dtype=pdt, pin_memory=True)
            self.v_host = torch.zeros(vshp, dtype=pdt, pin_memory=True)
            self.bm.enable_swap(host_blocks)

    def descriptor(self, shared_blocks: bool = False) -> N.PaCache:
        return ops.cache_desc(self.k_cache, self.v_cache, shared_blocks, scales=self.scales,
                              dtype=self.dtype)

    # ---- device operations ----------------------------------------------------------
    def write(self, k: torch.Tensor, v: torch.Tensor, slots) -> None:
        if isinstance(slots, np.ndarray):
            slots = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).to(self.device)
        ops.cache_write(self.k_cache, self.v_cache, k.to(self.device), v.to(self.device), slots,
                        scales=self.scales)

    def copy(self, pairs: np.ndarray) -> None:
        """Copy-on-write pairs from the block manager (in its blocks)."""
        pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
        if len(pairs) == 0:
            return
        pairs = self.bm.tile_pairs(pairs)                # block b = tiles 2 b, 2 b + 1
        ops.copy_blocks(self.k_cache, self.v_cache, torch.from_numpy(pairs).to(self.device),
                        pairs_host=pairs, scales=self.scales)

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

    def admit(self, sid: int, prompt: Sequence[int],
              token_kv: Callable[[int, int], Tuple[torch.Tensor, torch.Tensor]],
              tenant: int = 0) -> int:
        """Admit a request with automatic prefix caching.

        The sequence starts on the cached full blocks of ``prompt``; the other
        tokens get slots, their K/V ``token_kv(start, n)`` are stored, and their
        ids are committed so later requests can reuse the blocks they fill.  If
        the pool cannot hold the rest, the sequence is dropped again and
        OutOfBlocks propagates.  Returns the number of reused tokens (the
        caller computes attention for the others only)."""
        cached = self.bm.add_seq_cached(sid, prompt, tenant)
        n = len(prompt) - cached
        try:
            slots, cows = self.bm.append_tokens(sid, n)
        except N.OutOfBlocks:
            self.bm.free_seq(sid)
            raise
        self.copy(cows)
        k, v = token_kv(cached, n)
        self.write(k, v, slots)
        self.bm.commit_tokens(sid, list(prompt)[cached:])
        return cached

    # ---- swapping ----------------------------------------------------------------------
    def _swap(self, pairs: np.ndarray, direction: int) -> np.ndarray:
        if len(pairs):
            ops.swap_blocks(self.k_cache, self.v_cache, self.k_host, self.v_host, direction,
                            torch.from_numpy(np.ascontiguousarray(pairs)).to(self.device),
                            pairs_host=pairs, scales=self.scales)
        return pairs

    def swap_out(self, sids: Sequence[int]) -> np.ndarray:
        """Move the sequences' blocks to the host tier; the copies are enqueued on the
        current stream before anything later can reuse the released device blocks.
        Returns the (device, host) pairs."""
        return self._swap(self.bm.swap_out(sids), N.PA_SWAP_OUT)

    def swap_in(self, sids: Sequence[int]) -> np.ndarray:
        """Bring swapped-out sequences back into fresh device blocks; returns the (host,
        device) pairs."""
        return self._swap(self.bm.swap_in(sids), N.PA_SWAP_IN)

    def tables(self, sids: Sequence[int], max_blocks: int) -> Tuple[torch.Tensor, torch.Tensor, int]:
        """Device block tables and context lengths for ``sids``, plus the host max context."""
        tab, ctx = self.bm.pack(sids, max_blocks)
        return (torch.from_numpy(tab).to(self.device), torch.from_numpy(ctx).to(self.device),
                int(ctx.max()) if len(ctx) else 1)


class DecodeBatch:
    """Decode steps for a fixed list of sequences on one stream.

    ``step`` is one ``pa_decode_step`` call: the native block manager reserves
    the slots and packs the tables into a pinned staging buffer, then the
    copy-on-write copy and the fused store + decode are enqueued.  ``staging``
    says how the kernels get the staged values:

    * ``"mapped"``: they read the pinned buffer in place (no copy);
    * ``"upload"``: one copy to a device buffer on the step's stream;
    * ``"side"``: the copy runs on a side stream, so the copy of step i + 1
      overlaps the kernels of step i; the host waits for the copy before
      queueing the kernels (``last_host_waited``), so nothing stands between
      two steps' kernels on the stream.

    The default is "mapped" for a batch whose K/V can never pass 16 MiB (sequences x
    max_blocks_per_seq blocks; tiny batches are bound by the step's own latency, which
    a copy and its wait would lengthen) and "side" otherwise; ``zero_copy`` is the older
    switch (True: "mapped", False: "upload"), and an explicit ``staging`` wins over it.
    A ring of R pinned buffers (and, for "side", R device buffers; R even, up to 16 while
    they take at most 32 MiB of pinned memory) lets the host prepare later steps while
    earlier ones still read theirs.  Every R / 2 steps the step records one completion
    event on its stream; before a slot is reused the host waits for the first such
    event at or after the slot's last step, so no event sits between most pairs of
    kernels.  ``slots_d``, ``ctx_d``, ``tables_d`` and ``pairs_d`` view the last step's
    staged values.
    """

    def __init__(self, cache: PagedKVCache, sids: Sequence[int], num_heads: int, scale: float,
                 max_blocks_per_seq: int, stream: Optional[torch.cuda.Stream] = None,
                 zero_copy: Optional[bool] = None, staging: Optional[str] = None):
        self.cache = cache
        self.sids = np.ascontiguousarray(np.asarray(sids, dtype=np.int64))
        self.B = B = len(self.sids)
        self.H = num_heads
        self.scale = float(scale)
        self.max_blocks = max_blocks_per_seq
        self.stream = stream if stream is not None else torch.cuda.current_stream(cache.device)
        if staging is not None:
            mode = staging
        elif zero_copy is None:
            tile_bytes = 16 * cache.head_dim * (1 if cache.fp8 else cache.k_cache.element_size())
            kv_max = 2 * B * max_blocks_per_seq * cache.num_kv_heads * tile_bytes
            mode = "mapped" if kv_max <= _MAPPED_MAX_KV_BYTES else "side"
        else:
            mode = "mapped" if zero_copy else "upload"
        if mode not in ("mapped", "upload", "side"):
            raise ValueError(f"staging must be 'mapped', 'upload' or 'side', not {mode!r}")
        self.staging = mode
        self.zero_copy = mode == "mapped"
        dev = cache.device
        lib = N.lib()
        self._lib = lib
        self._bytes = int(lib.pa_decode_step_staging_bytes(B, max_blocks_per_seq))
        ring = _ring_slots(self._bytes)
        self._ring = ring
        # 256-byte aligned regions carved from slightly larger allocations
        self._pinned_raw = [torch.empty(self._bytes + _ALIGN, dtype=torch.uint8, pin_memory=True)
                            for _ in range(ring)]
        self._pinned = [self._aligned(t) for t in self._pinned_raw]
        self._marks = _CompletionMarks(ring // 2, torch.cuda.Event, lambda e: e.record(self.stream),
                                       lambda e: e.synchronize(), lambda: self.stream.synchronize())
        n_dev = ring if mode == "side" else 1
        self._dev_raw = [torch.empty(self._bytes + _ALIGN, dtype=torch.uint8, device=dev)
                         for _ in range(n_dev)]
        self._dev = [self._aligned(t) for t in self._dev_raw]
        self._copy_stream = None
        self._copied = []
        if mode == "side":
            self._copy_stream = torch.cuda.Stream(dev)       # default priority
            self._copied = [torch.cuda.Event() for _ in range(ring)]
            for e in self._copied:
                e.record(self._copy_stream)                  # creates the handles
        off_ctx = _round(8 * B)
        off_tab = off_ctx + _round(4 * B)
        off_pairs = off_tab + _round(4 * B * max_blocks_per_seq)
        self._offs = (0, off_ctx, off_tab, off_pairs)
        self._last_buf = None
        self._last_dev = 0
        self._dev_current = True
        self.out = torch.empty((B, num_heads, cache.head_dim), dtype=cache.dtype, device=dev)
        self.workspace = ops.alloc_workspace(B, num_heads, cache.head_dim,
                                             max_blocks_per_seq * N.BLOCK_SIZE, dev)
        self._desc = cache.descriptor()
        self._info = N.PaStepInfo()
        self._sids_ptr = self.sids.ctypes.data
        self._device = cache.k_cache.device
        self._kv_shape = (B, cache.num_kv_heads, cache.head_dim)
        self._q_shape = (B, num_heads, cache.head_dim)
        self._i = 0
        self.last_max_ctx = 0
        self.last_grouped = False
        self.last_host_waited = False
        self.last_pairs = np.zeros((0, 2), dtype=np.int32)
        # First uses cost tens of microseconds each (an event's creation, a buffer's first
        # copy); take them here rather than in the first pass over the ring.
        self._marks.prime(3)
        if mode != "mapped":
            cs = self._copy_stream if mode == "side" else self.stream
            with torch.cuda.stream(cs):
                for i in range(ring):
                    d = self._dev[i if mode == "side" else 0]
                    d.copy_(self._pinned[i], non_blocking=True)
        torch.cuda.synchronize(dev)

    def _staged_dev(self) -> torch.Tensor:
        """The device buffer holding the last step's staged values (copied there on
        demand in "mapped" mode)."""
        d = self._dev[self._last_dev]
        if not self._dev_current and self._last_buf is not None:
            d.copy_(self._pinned[self._last_buf], non_blocking=False)
            self._dev_current = True
        return d

    @property
    def slots_d(self) -> torch.Tensor:
        return self._staged_dev()[0:8 * self.B].view(torch.int64)

    @property
    def ctx_d(self) -> torch.Tensor:
        o = self._offs[1]
        return self._staged_dev()[o:o + 4 * self.B].view(torch.int32)

    @property
    def tables_d(self) -> torch.Tensor:
        o = self._offs[2]
        n = 4 * self.B * self.max_blocks
        return self._staged_dev()[o:o + n].view(torch.int32).view(self.B, self.max_blocks)

    @property
    def pairs_d(self) -> torch.Tensor:
        o = self._offs[3]
        return self._staged_dev()[o:o + 8 * self.B].view(torch.int32).view(self.B, 2)

    @staticmethod
    def _aligned(t: torch.Tensor) -> torch.Tensor:
        pad = (-t.data_ptr()) % _ALIGN
        return t[pad:]

    def step(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
             attn_events: Optional[Tuple[torch.cuda.Event, torch.cuda.Event]] = None) -> torch.Tensor:
        """One decode step (host reservation included).  Returns the output tensor (reused).

        k_new, v_new: [B, Hkv, D] of the step's new tokens; q: [B, H, D]; all
        contiguous device tensors of the cache dtype.  ``attn_events``, if given,
        take the start and end of the attention kernel (attached to its dispatch).
        """
        for t, shape in ((k_new, self._kv_shape), (v_new, self._kv_shape), (q, self._q_shape)):
            if (t.dtype != self.cache.dtype or t.device != self._device
                    or tuple(t.shape) != shape or not t.is_contiguous()):
                raise ValueError(f"step inputs: need contiguous {self.cache.dtype} tensors of shape "
                                 f"{shape} on {self._device}")
        if attn_events is not None:
            for e in attn_events:
                if not e.cuda_event:
                    e.record(self.stream)        # creates the handle
        i = self._i
        buf = i % self._ring
        self._i += 1
        # The slot's last reader (the kernels, or in "side" mode the copy, of step
        # i - ring) has finished: the slot's pinned and device buffers may be rewritten.
        self._marks.wait(i - self._ring)
        pin = self._pinned[buf]
        ev = (None, None) if attn_events is None else (attn_events[0].cuda_event,
                                                       attn_events[1].cuda_event)
        ws = self.workspace
        side = self._copy_stream is not None
        di = buf if side else 0
        N.check(self._lib.pa_decode_step(
            self.cache.bm._h, C.byref(self._desc), self.B, self._sids_ptr, k_new.data_ptr(),
            v_new.data_ptr(), q.data_ptr(), self.H, self.scale, self.out.data_ptr(),
            ws.data_ptr(), ws.numel(), pin.data_ptr(),
            None if self.zero_copy else self._dev[di].data_ptr(), self._bytes,
            self.max_blocks, ev[0], ev[1], C.byref(self._info),
            self._copy_stream.cuda_stream if side else None,
            self._copied[buf].cuda_event if side else None, self.stream.cuda_stream),
            "pa_decode_step")
        self._marks.after(i)
        self._last_buf = buf
        self._last_dev = di
        self._dev_current = not self.zero_copy
        n_cow = self._info.num_cow
        if n_cow:
            o = self._offs[3]
            self.last_pairs = pin[o:o + 8 * n_cow].view(torch.int32).view(n_cow, 2).numpy().copy()
        else:
            self.last_pairs = np.zeros((0, 2), dtype=np.int32)
        self.last_max_ctx = self._info.max_context_len
        self.last_grouped = bool(self._info.grouped)
        self.last_host_waited = bool(self._info.host_waited)
        return self.out
