"""Python handle on the native host block manager (pa_bm_* in libpa.so)."""

from __future__ import annotations

import ctypes as C
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from . import _native as N


def _ptr(a: np.ndarray) -> C.c_void_p:
    return C.c_void_p(a.ctypes.data)


class BlockManager:
    """Free list, reference counts, fork and copy-on-write, and (with prefix_caching)
    automatic prefix caching; pa.h states the policies."""

    def __init__(self, num_blocks: int, block_size: int = N.BLOCK_SIZE,
                 free_order: Optional[Sequence[int]] = None, prefix_caching: bool = False):
        self._lib = N.lib()
        h = C.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if order.shape != (num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
        N.check(self._lib.pa_bm_create(num_blocks, block_size,
                                       None if order is None else _ptr(order), C.byref(h)),
                "pa_bm_create")
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size
        if prefix_caching:
            N.check(self._lib.pa_bm_enable_prefix_cache(self._h), "pa_bm_enable_prefix_cache")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pa_bm_destroy(h)
            self._h = None

    def add_seq(self, sid: int) -> None:
        N.check(self._lib.pa_bm_add_seq(self._h, sid), "pa_bm_add_seq")

    def append(self, sid: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        slot = C.c_int64()
        s, d = C.c_int32(), C.c_int32()
        N.check(self._lib.pa_bm_append(self._h, sid, C.byref(slot), C.byref(s), C.byref(d)),
                "pa_bm_append")
        return slot.value, ((s.value, d.value) if s.value >= 0 else None)

    def append_batch(self, sids: Iterable[int], slots_out: Optional[np.ndarray] = None
                     ) -> Tuple[np.ndarray, np.ndarray]:
        """One token for each sequence.  Returns (slots int64[n], cow pairs int32[k, 2])."""
        ids = np.ascontiguousarray(np.asarray(list(sids) if not isinstance(sids, np.ndarray)
                                              else sids, dtype=np.int64))
        n = ids.shape[0]
        slots = slots_out if slots_out is not None else np.empty(n, dtype=np.int64)
        cows = np.empty((max(n, 1), 2), dtype=np.int32)
        nc = C.c_int32()
        N.check(self._lib.pa_bm_append_batch(self._h, n, _ptr(ids), _ptr(slots), _ptr(cows),
                                             max(n, 1), C.byref(nc)), "pa_bm_append_batch")
        return slots, cows[:nc.value]

    def append_tokens(self, sid: int, count: int) -> Tuple[np.ndarray, np.ndarray]:
        slots = np.empty(max(count, 1), dtype=np.int64)
        cows = np.empty((max(count, 1), 2), dtype=np.int32)
        nc = C.c_int32()
        N.check(self._lib.pa_bm_append_tokens(self._h, sid, count, _ptr(slots), _ptr(cows),
                                              max(count, 1), C.byref(nc)), "pa_bm_append_tokens")
        return slots[:count], cows[:nc.value]

    def fork(self, parent: int, child: int) -> None:
        N.check(self._lib.pa_bm_fork(self._h, parent, child), "pa_bm_fork")

    def free_seq(self, sid: int) -> None:
        N.check(self._lib.pa_bm_free_seq(self._h, sid), "pa_bm_free_seq")

    def seq_len(self, sid: int) -> int:
        n = C.c_int64()
        N.check(self._lib.pa_bm_seq_len(self._h, sid, C.byref(n)), "pa_bm_seq_len")
        return n.value

    def block_table(self, sid: int) -> List[int]:
        n = C.c_int32()
        N.check(self._lib.pa_bm_block_table(self._h, sid, None, 0, C.byref(n)), "pa_bm_block_table")
        out = np.empty(max(n.value, 1), dtype=np.int32)
        N.check(self._lib.pa_bm_block_table(self._h, sid, _ptr(out), n.value, C.byref(n)),
                "pa_bm_block_table")
        return out[:n.value].tolist()

    def pack(self, sids: Sequence[int], max_blocks: int, tables_out: Optional[np.ndarray] = None,
             ctx_out: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Block tables int32[n, max_blocks] (unused -1) and context lengths int32[n]."""
        ids = np.ascontiguousarray(np.asarray(sids, dtype=np.int64))
        n = ids.shape[0]
        tables = tables_out if tables_out is not None else np.empty((n, max_blocks), dtype=np.int32)
        ctx = ctx_out if ctx_out is not None else np.empty(n, dtype=np.int32)
        N.check(self._lib.pa_bm_pack(self._h, n, _ptr(ids), _ptr(tables), max_blocks, _ptr(ctx)),
                "pa_bm_pack")
        return tables, ctx

    def step(self, sids: Sequence[int], max_blocks: int):
        """pa_bm_step: one token for each sequence, then pack.

        Returns (slots int64[n], cow pairs int32[k, 2], tables int32[n, max_blocks],
        context lengths int32[n], longest context).
        """
        ids = np.ascontiguousarray(np.asarray(sids, dtype=np.int64))
        n = ids.shape[0]
        slots = np.empty(max(n, 1), dtype=np.int64)
        cows = np.empty((max(n, 1), 2), dtype=np.int32)
        tables = np.empty((max(n, 1), max_blocks), dtype=np.int32)
        ctx = np.empty(max(n, 1), dtype=np.int32)
        nc, mx = C.c_int32(), C.c_int32()
        N.check(self._lib.pa_bm_step(self._h, n, _ptr(ids), _ptr(slots), _ptr(cows), max(n, 1),
                                     C.byref(nc), _ptr(tables), max_blocks, _ptr(ctx), C.byref(mx)),
                "pa_bm_step")
        return slots[:n], cows[:nc.value], tables[:n], ctx[:n], mx.value

    def refcount(self, blk: int) -> int:
        r = C.c_int32()
        N.check(self._lib.pa_bm_refcount(self._h, blk, C.byref(r)), "pa_bm_refcount")
        return r.value

    def free_list(self) -> List[int]:
        n = C.c_int32()
        out = np.empty(self.num_blocks, dtype=np.int32)
        N.check(self._lib.pa_bm_free_list(self._h, _ptr(out), self.num_blocks, C.byref(n)),
                "pa_bm_free_list")
        return out[:n.value].tolist()

    def tile_pairs(self, pairs) -> np.ndarray:
        """Copy-on-write pairs of manager blocks as pairs of pool tiles (pa_bm_tile_pairs)."""
        p = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        cap = 2 * max(1, p.shape[0])
        out = np.empty((cap, 2), dtype=np.int32)
        n = C.c_int32()
        N.check(self._lib.pa_bm_tile_pairs(self._h, _ptr(p), p.shape[0], _ptr(out), cap,
                                           C.byref(n)), "pa_bm_tile_pairs")
        return out[:n.value]

    def stats(self) -> dict:
        st = N.PaBmStats()
        N.check(self._lib.pa_bm_stats_get(self._h, C.byref(st)), "pa_bm_stats_get")
        return {f: getattr(st, f) for f, _ in N.PaBmStats._fields_}

    # -- automatic prefix caching ----------------------------------------------------
    def add_seq_cached(self, sid: int, prompt, tenant: int = 0) -> int:
        """New sequence holding the cached full blocks of ``prompt``; returns their tokens."""
        ids = np.ascontiguousarray(np.asarray(prompt, dtype=np.int32).reshape(-1))
        cached = C.c_int32()
        N.check(self._lib.pa_bm_add_seq_cached(self._h, sid, tenant, _ptr(ids), ids.shape[0],
                                               C.byref(cached)), "pa_bm_add_seq_cached")
        return cached.value

    def admit_batch(self, sids: Sequence[int], tokens, offsets, tenants=None,
                    slots_out: Optional[np.ndarray] = None):
        """pa_bm_admit_batch: prompts tokens[offsets[i]:offsets[i+1]] (int32, int64[n+1]).

        Returns (cached int32[n], slots int64[new tokens], admitted).  On running out of
        blocks, OutOfBlocks is raised after the admitted prefix of the list stays admitted;
        its ``admitted`` attribute says how many."""
        s = np.ascontiguousarray(np.asarray(sids, dtype=np.int64))
        n = s.shape[0]
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
        if off.shape != (n + 1,):
            raise ValueError("offsets must have n + 1 entries")
        ten = None
        if tenants is not None:
            ten = np.ascontiguousarray(np.asarray(tenants, dtype=np.int64))
        total = int(off[-1] - off[0]) if n else 0
        slots = slots_out if slots_out is not None else np.empty(max(total, 1), dtype=np.int64)
        cached = np.zeros(max(n, 1), dtype=np.int32)
        adm = C.c_int32()
        st = self._lib.pa_bm_admit_batch(self._h, n, _ptr(s), None if ten is None else _ptr(ten),
                                         _ptr(tok) if tok.size else None, _ptr(off), _ptr(cached),
                                         _ptr(slots), slots.shape[0], C.byref(adm))
        try:
            N.check(st, "pa_bm_admit_batch")
        except N.OutOfBlocks as e:
            e.admitted = adm.value
            raise
        k = adm.value
        new = int((np.diff(off[:k + 1]) - cached[:k]).sum()) if k else 0
        return cached[:n], slots[:new], k

    def commit_tokens(self, sid: int, token_ids) -> None:
        ids = np.ascontiguousarray(np.asarray(token_ids, dtype=np.int32).reshape(-1))
        N.check(self._lib.pa_bm_commit_tokens(self._h, sid, _ptr(ids), ids.shape[0]),
                "pa_bm_commit_tokens")

    def commit_batch(self, sids: Sequence[int], token_ids) -> None:
        s = np.ascontiguousarray(np.asarray(sids, dtype=np.int64))
        ids = np.ascontiguousarray(np.asarray(token_ids, dtype=np.int32).reshape(-1))
        if ids.shape[0] != s.shape[0]:
            raise ValueError("one token id per sequence")
        N.check(self._lib.pa_bm_commit_batch(self._h, s.shape[0], _ptr(s), _ptr(ids)),
                "pa_bm_commit_batch")

    def reset_prefix_cache(self) -> None:
        N.check(self._lib.pa_bm_prefix_cache_reset(self._h), "pa_bm_prefix_cache_reset")

    def prefix_stats(self) -> dict:
        st = N.PaBmPrefixStats()
        N.check(self._lib.pa_bm_prefix_stats_get(self._h, C.byref(st)), "pa_bm_prefix_stats_get")
        return {f: getattr(st, f) for f, _ in N.PaBmPrefixStats._fields_}

    def _block_list(self, fn) -> List[int]:
        n = C.c_int32()
        out = np.empty(self.num_blocks, dtype=np.int32)
        N.check(getattr(self._lib, fn)(self._h, _ptr(out), self.num_blocks, C.byref(n)), fn)
        return out[:n.value].tolist()

    def evictable_blocks(self) -> List[int]:
        """Evictable blocks, next to evict first."""
        return self._block_list("pa_bm_evictable_list")

    def cached_blocks(self) -> List[int]:
        """Blocks in the prefix index, ascending."""
        return self._block_list("pa_bm_cached_list")

    # -- swapping to a host tier -------------------------------------------------------
    def enable_swap(self, num_host_blocks: int, host_free_order: Optional[Sequence[int]] = None) -> None:
        order = None
        if host_free_order is not None:
            order = np.ascontiguousarray(np.asarray(host_free_order, dtype=np.int32))
        N.check(self._lib.pa_bm_enable_swap(self._h, num_host_blocks,
                                            None if order is None else _ptr(order)),
                "pa_bm_enable_swap")
        self.num_host_blocks = num_host_blocks

    def _swap(self, fn: str, sids: Sequence[int]) -> np.ndarray:
        ids = np.ascontiguousarray(np.asarray(list(sids), dtype=np.int64))
        cap = 0
        for sid in ids.tolist():                       # table lengths bound the distinct blocks
            cap += self.seq_blocks(sid)
        pairs = np.empty((max(cap, 1), 2), dtype=np.int32)
        n = C.c_int32()
        N.check(getattr(self._lib, fn)(self._h, ids.shape[0], _ptr(ids), _ptr(pairs), max(cap, 1),
                                       C.byref(n)), fn)
        return pairs[:n.value]

    def swap_out(self, sids: Sequence[int]) -> np.ndarray:
        """(device block, host block) pairs to copy out, int32 [k, 2]."""
        return self._swap("pa_bm_swap_out", sids)

    def swap_in(self, sids: Sequence[int]) -> np.ndarray:
        """(host block, device block) pairs to copy in, int32 [k, 2]."""
        return self._swap("pa_bm_swap_in", sids)

    def is_swapped(self, sid: int) -> bool:
        r = C.c_int32()
        N.check(self._lib.pa_bm_is_swapped(self._h, sid, C.byref(r)), "pa_bm_is_swapped")
        return bool(r.value)

    def seq_blocks(self, sid: int) -> int:
        """Blocks a sequence holds in its current tier (0 for an unknown sequence)."""
        n = C.c_int64()
        if self._lib.pa_bm_seq_len(self._h, sid, C.byref(n)) != N.PA_OK:
            return 0
        return -(-n.value // self.block_size)

    def host_table(self, sid: int) -> List[int]:
        n = C.c_int32()
        N.check(self._lib.pa_bm_host_table(self._h, sid, None, 0, C.byref(n)), "pa_bm_host_table")
        out = np.empty(max(n.value, 1), dtype=np.int32)
        N.check(self._lib.pa_bm_host_table(self._h, sid, _ptr(out), n.value, C.byref(n)),
                "pa_bm_host_table")
        return out[:n.value].tolist()

    def host_refcount(self, blk: int) -> int:
        r = C.c_int32()
        N.check(self._lib.pa_bm_host_refcount(self._h, blk, C.byref(r)), "pa_bm_host_refcount")
        return r.value

    def host_free_list(self) -> List[int]:
        n = C.c_int32()
        out = np.empty(max(getattr(self, "num_host_blocks", 0), 1), dtype=np.int32)
        N.check(self._lib.pa_bm_host_free_list(self._h, _ptr(out), out.shape[0], C.byref(n)),
                "pa_bm_host_free_list")
        return out[:n.value].tolist()
