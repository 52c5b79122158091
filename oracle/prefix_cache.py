"""Reference automatic prefix caching over the block manager.  TEST INFRASTRUCTURE ONLY.

What the pages fix:

* A request whose leading tokens equal those of an earlier request reuses the
  KV blocks already computed for them and skips their prefill; the match is
  found automatically ("vLLM 核心概念", section 前缀缓存（Prefix Caching） and its
  part on automatic matching; "PagedAttention 实战", section "Prefix Caching：
  让相同前缀不要反复算").
* Reuse is by pointing the new request's logical blocks at the same physical
  blocks; the system keeps the block references, a hash index, the blocks'
  lifecycle and an eviction policy ("理解 vLLM PagedAttention", section 六).
* It needs cache space, hit-rate statistics, an eviction policy (LRU, cost,
  or hit prediction) and multi-tenant isolation, and caches must be dropped
  when the model changes ("PagedAttention 实战", the same section and its
  fifth step on eviction and isolation).

Readings where the pages leave the rule open (each also in the design notes):

* Unit of reuse: a full block.  The K/V of a token depend on every token
  before it, so a block is identified by the whole prefix through its last
  token (and by the tenant), never by its own 16 tokens alone.  Here the index
  is literally a dict from (tenant, full prefix) to the physical block.
* A block enters the index when its 16th token id is committed (the caller
  commits ids for slots it has already appended and written), if its prefix
  is not indexed yet and the block is not indexed under another prefix.  An
  indexed block is full, hence never written again.
* Matching: a new request walks its prompt's full blocks from the first and
  reuses each whose prefix is indexed, stopping at the first miss; at most
  floor((n - 1) / 16) blocks, so at least one prompt token is left for the
  model to compute.  A hit takes a reference on the block.
* Lifecycle: an indexed block whose reference count drops to zero keeps its
  contents and becomes evictable; other blocks go back to the free stack.
* Eviction is LRU: allocation pops the free stack first; only when it is empty
  does it evict the evictable block released longest ago (release times are
  one counter, advanced per released block, so a sequence's tail blocks,
  released first, go before its head blocks).  Evicting removes the block's
  index entry.
* Tenants: a prefix only matches blocks committed under the same tenant id.
* Invalidation (a model change): every index entry is dropped; evictable blocks
  are pushed onto the free stack oldest first.
* Statistics: requests, full blocks looked up, blocks hit, evictions.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

from .block_manager import RefBlockManager


class RefPrefixCache(RefBlockManager):
    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order: Optional[Sequence[int]] = None):
        super().__init__(num_blocks, block_size, free_order)
        self._index: Dict[Tuple[int, Tuple[int, ...]], int] = {}   # (tenant, prefix) -> block
        self._block_key: Dict[int, Tuple[int, Tuple[int, ...]]] = {}
        self._evictable: Dict[int, int] = {}                        # block -> release time
        self._clock = 0
        self._tenant: Dict[int, int] = {}
        self._committed: Dict[int, List[int]] = {}                  # token ids, in order
        self.requests = 0
        self.query_blocks = 0
        self.hit_blocks = 0
        self.evictions = 0

    # -- sequences -----------------------------------------------------------------
    def add_seq(self, sid: int, tenant: int = 0) -> None:
        super().add_seq(sid)
        self._tenant[sid] = tenant
        self._committed[sid] = []

    def add_seq_cached(self, sid: int, prompt: Sequence[int], tenant: int = 0) -> int:
        """Create a sequence holding the longest indexed prefix of ``prompt`` (full blocks,
        at most floor((n-1)/16)); returns the number of tokens it now holds."""
        self.add_seq(sid, tenant)
        prompt = [int(t) for t in prompt]
        bs = self.block_size
        most = self._lookup_limit(len(prompt))
        hits = 0
        for j in range(most):
            blk = self._index.get(self._key(tenant, prompt[:bs * (j + 1)]))
            if blk is None:
                break
            if self._ref[blk] == 0:
                del self._evictable[blk]
            self._ref[blk] += 1
            self._tables[sid].append(blk)
            hits += 1
        self._lens[sid] = bs * hits
        self._committed[sid] = prompt[:bs * hits]
        self.requests += 1
        self.query_blocks += most
        self.hit_blocks += hits
        return bs * hits

    def commit_tokens(self, sid: int, token_ids: Sequence[int]) -> None:
        """Token ids of the sequence's next appended-but-uncommitted slots, in order."""
        done = self._committed[sid]
        if len(done) + len(token_ids) > self._lens[sid]:
            raise ValueError("commit beyond the appended tokens")
        bs = self.block_size
        for t in token_ids:
            done.append(int(t))
            if len(done) % bs == 0:
                blk = self._tables[sid][len(done) // bs - 1]
                key = self._key(self._tenant[sid], done)
                if key not in self._index and blk not in self._block_key:
                    self._index[key] = blk
                    self._block_key[blk] = key

    def commit_batch(self, sids: Sequence[int], token_ids: Sequence[int]) -> None:
        """One token id for each of several distinct sequences; all or nothing."""
        if len(set(sids)) != len(sids) or len(sids) != len(token_ids):
            raise ValueError("one id for each distinct sequence")
        for sid in sids:
            if self._lens[sid] - len(self._committed[sid]) < 1:
                raise ValueError("commit beyond the appended tokens")
        for sid, t in zip(sids, token_ids):
            self.commit_tokens(sid, [t])

    def fork(self, parent: int, child: int) -> None:
        super().fork(parent, child)
        self._tenant[child] = self._tenant[parent]
        self._committed[child] = list(self._committed[parent])

    def free_seq(self, sid: int) -> None:
        super().free_seq(sid)
        del self._tenant[sid]
        del self._committed[sid]

    def reset(self) -> None:
        """Drop every index entry (a model change); evictable blocks return to the free
        stack, oldest release first."""
        for blk in sorted(self._evictable, key=self._evictable.get):
            self._free.append(blk)
        self._evictable.clear()
        self._index.clear()
        self._block_key.clear()

    def _key(self, tenant: int, prefix: Sequence[int]) -> Tuple[int, Tuple[int, ...]]:
        """Index key of the block that ends ``prefix``: the tenant and the whole prefix."""
        return (tenant, tuple(prefix))

    def _lookup_limit(self, n: int) -> int:
        """Full blocks of an n-token prompt that may be reused: one token stays to compute."""
        return (n - 1) // self.block_size if n > 0 else 0

    # -- where blocks come from and go to ---------------------------------------------
    def _available(self) -> int:
        return len(self._free) + len(self._evictable)

    def _take(self) -> int:
        if self._free:
            return self._free.pop()
        blk = min(self._evictable, key=self._evictable.get)
        del self._evictable[blk]
        del self._index[self._block_key.pop(blk)]
        self.evictions += 1
        return blk

    def _release(self, blk: int) -> None:
        if blk in self._block_key:
            self._evictable[blk] = self._clock
            self._clock += 1
        else:
            self._free.append(blk)

    # -- queries ---------------------------------------------------------------------
    def cached_blocks(self) -> List[int]:
        """Indexed blocks, ascending."""
        return sorted(self._block_key)

    def evictable_blocks(self) -> List[int]:
        """Evictable blocks, next to evict first."""
        return sorted(self._evictable, key=self._evictable.get)

    def committed(self, sid: int) -> List[int]:
        return list(self._committed[sid])

    def prefix_stats(self) -> Dict[str, int]:
        return {"requests": self.requests, "query_blocks": self.query_blocks,
                "hit_blocks": self.hit_blocks, "cached_blocks": len(self._block_key),
                "evictable_blocks": len(self._evictable), "evictions": self.evictions}
