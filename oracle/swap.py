"""Reference GPU <-> host block swapping.  TEST INFRASTRUCTURE ONLY.

What the pages fix: KV blocks live in a memory hierarchy; GPU memory holds the
active requests' caches, blocks that do not fit spill to CPU memory and are
swapped back in when needed, so a batch larger than GPU memory can be served
("vLLM 核心概念", section 内存层次结构, and its remark on KV cache offloading);
preemption is the fallback when resources run short ("理解 vLLM PagedAttention",
section 五).

Readings where the pages leave the rule open (each also in the design notes):

* The host tier is a second pool of blocks of the same shape with its own LIFO
  free stack (starting as a given permutation, first entry popped first) and
  reference counts.
* Swapping out a list of sequences moves all of them at once: every distinct
  device block they reference (in order of first appearance: sequence order,
  then logical order) gets one host block, so blocks shared among the listed
  sequences stay shared; the (device, host) pairs say what to copy.  Then the
  listed sequences drop their device references, sequence by sequence, last
  logical block first (as when a sequence ends).  A block still referenced by
  a sequence that stays resident keeps its device copy.
* Swapping in is the mirror image: one device block (taken as an append takes
  one, so cached blocks may be evicted) per distinct host block, (host, device)
  pairs to copy, then the host references are dropped the same way.
* Both are all or nothing: not enough free blocks in the target tier raises
  OutOfBlocks and changes nothing.
* A swapped-out sequence cannot grow, fork or commit; it can be freed, which
  releases its host blocks.  Its prefix-cache state (tenant, committed ids)
  travels with it.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

from .block_manager import OutOfBlocks
from .prefix_cache import RefPrefixCache


class RefSwapManager(RefPrefixCache):
    def __init__(self, num_blocks: int, num_host_blocks: int, block_size: int = 16,
                 free_order: Optional[Sequence[int]] = None,
                 host_free_order: Optional[Sequence[int]] = None):
        super().__init__(num_blocks, block_size, free_order)
        horder = list(range(num_host_blocks)) if host_free_order is None else list(host_free_order)
        if sorted(horder) != list(range(num_host_blocks)):
            raise ValueError("host_free_order must be a permutation of range(num_host_blocks)")
        self.num_host_blocks = num_host_blocks
        self._hfree: List[int] = list(reversed(horder))
        self._href: List[int] = [0] * num_host_blocks
        self._swapped: Dict[int, Tuple[List[int], int]] = {}   # sid -> (host table, length)

    @staticmethod
    def _distinct(tables: Sequence[Sequence[int]]) -> List[int]:
        seen, order = set(), []
        for t in tables:
            for b in t:
                if b not in seen:
                    seen.add(b)
                    order.append(b)
        return order

    def _check(self, sids, where) -> None:
        if len(set(sids)) != len(sids):
            raise ValueError("a list names each sequence at most once")
        for sid in sids:
            if sid not in where:
                raise KeyError(f"sequence {sid} is not where the call expects it")

    def swap_out(self, sids: Sequence[int]) -> List[Tuple[int, int]]:
        """Move the sequences to the host tier; returns (device block, host block) pairs."""
        sids = list(sids)
        self._check(sids, self._tables)
        tables = [self._tables[s] for s in sids]
        distinct = self._distinct(tables)
        if len(distinct) > len(self._hfree):
            raise OutOfBlocks(f"swap-out needs {len(distinct)} host blocks, {len(self._hfree)} free")
        to_host = {}
        for d in distinct:
            to_host[d] = self._hfree.pop()
        for sid, table in zip(sids, tables):
            htable = [to_host[d] for d in table]
            for h in htable:
                self._href[h] += 1
            self._swapped[sid] = (htable, self._lens[sid])
            del self._tables[sid]
            del self._lens[sid]
        for table in tables:
            for d in reversed(table):
                self._ref[d] -= 1
                if self._ref[d] == 0:
                    self._release(d)
        return [(d, to_host[d]) for d in distinct]

    def swap_in(self, sids: Sequence[int]) -> List[Tuple[int, int]]:
        """Bring the sequences back; returns (host block, device block) pairs."""
        sids = list(sids)
        self._check(sids, self._swapped)
        htables = [self._swapped[s][0] for s in sids]
        distinct = self._distinct(htables)
        if len(distinct) > self._available():
            raise OutOfBlocks(f"swap-in needs {len(distinct)} blocks, {self._available()} available")
        to_dev = {}
        for h in distinct:
            d = self._take()
            self._ref[d] = 0
            to_dev[h] = d
        for sid, htable in zip(sids, htables):
            table = [to_dev[h] for h in htable]
            for d in table:
                self._ref[d] += 1
            self._tables[sid] = table
            self._lens[sid] = self._swapped.pop(sid)[1]
        for htable in htables:
            for h in reversed(htable):
                self._href[h] -= 1
                if self._href[h] == 0:
                    self._hfree.append(h)
        return [(h, to_dev[h]) for h in distinct]

    def free_seq(self, sid: int) -> None:
        if sid in self._swapped:
            htable, _ = self._swapped.pop(sid)
            for h in reversed(htable):
                self._href[h] -= 1
                if self._href[h] == 0:
                    self._hfree.append(h)
            self._tenant.pop(sid, None)
            self._committed.pop(sid, None)
        else:
            super().free_seq(sid)

    # -- queries ---------------------------------------------------------------------
    def is_swapped(self, sid: int) -> bool:
        return sid in self._swapped

    def host_table(self, sid: int) -> List[int]:
        return list(self._swapped[sid][0])

    def host_refcount(self, h: int) -> int:
        return self._href[h]

    def host_free_list(self) -> List[int]:
        """Free host blocks, next-to-pop first."""
        return list(reversed(self._hfree))
