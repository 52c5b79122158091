"""Reference block manager in plain Python.  TEST INFRASTRUCTURE ONLY.

Behaviour and where the pages fix it:

* A global pool of fixed-size blocks: a sequence takes blocks from it, appends
  blocks as it grows, returns them when it ends, and several sequences may
  point logical blocks at the same physical block ("理解 vLLM PagedAttention",
  section 三).
* Allocation is on demand: a new block is taken exactly when the sequence's
  last block is full, the first token included; a 64-token sequence ends with
  four blocks ("vLLM 核心概念", sections "逻辑视图与物理视图分离" and "按需分配";
  "理解 vLLM PagedAttention", section 四).  Waste is confined to the last block.
* Sharing and copy-on-write: forked sequences (beam search, parallel
  sampling) point at the parent's blocks; a new block is allocated only when
  later tokens diverge ("理解 vLLM PagedAttention", section 六; "vLLM 核心概念",
  section "内存共享").

Readings where the pages are silent (each also listed in the design notes):

* Free list: a LIFO stack.  It starts as a given permutation ``free_order`` of
  [0, num_blocks) and pops free_order[0] first; a freed block is pushed on top.
* Release: a finished sequence drops one reference from each of its blocks,
  last logical block first; a block whose count reaches zero is pushed, so the
  first logical block ends up on top.
* Copy-on-write: only a shared (refcount > 1), partially filled last block
  that is about to be written is copied.  The appending sequence gets a fresh
  block and the pair (old, new) is reported; the old block loses one
  reference.  The last remaining sharer writes in place.  Full shared blocks
  are never copied.
* An append that finds no free block fails and changes nothing; a batch of
  appends either succeeds as a whole or changes nothing.
"""

from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple


class OutOfBlocks(Exception):
    pass


class RefBlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._free: List[int] = list(reversed(order))   # top of stack = end of list
        self._ref: List[int] = [0] * num_blocks
        self._tables: Dict[int, List[int]] = {}
        self._lens: Dict[int, int] = {}

    # -- sequences ---------------------------------------------------------------
    def add_seq(self, sid: int) -> None:
        if sid in self._tables:
            raise KeyError(f"sequence {sid} exists")
        self._tables[sid] = []
        self._lens[sid] = 0

    def _needs_block(self, sid: int, pending_drop: Dict[int, int]) -> bool:
        n = self._lens[sid]
        if n % self.block_size == 0:
            return True
        last = self._tables[sid][-1]
        return self._ref[last] - pending_drop.get(last, 0) > 1

    def append(self, sid: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of sequence ``sid``'s next token.  Returns (slot, cow pair or None)."""
        slots, cows = self.append_batch([sid])
        return slots[0], (cows[0] if cows else None)

    def append_batch(self, sids: Iterable[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One token for each sequence, in order; all-or-nothing."""
        sids = list(sids)
        for sid in sids:
            if sid not in self._tables:
                raise KeyError(f"no sequence {sid}")
        if len(set(sids)) != len(sids):
            raise ValueError("a batch names each sequence at most once")
        # count the blocks the batch takes, with the reference drops earlier CoWs make
        drop: Dict[int, int] = {}
        need = 0
        for sid in sids:
            if self._needs_block(sid, drop):
                need += 1
                if self._lens[sid] % self.block_size:
                    last = self._tables[sid][-1]
                    drop[last] = drop.get(last, 0) + 1
        if need > self._available():
            raise OutOfBlocks(f"batch needs {need} blocks, {self._available()} available")
        slots, cows = [], []
        for sid in sids:
            table = self._tables[sid]
            n = self._lens[sid]
            off = n % self.block_size
            if off == 0:
                blk = self._take()
                self._ref[blk] = 1
                table.append(blk)
            else:
                last = table[-1]
                if self._ref[last] > 1:
                    blk = self._take()
                    self._ref[blk] = 1
                    self._ref[last] -= 1
                    table[-1] = blk
                    cows.append((last, blk))
                else:
                    blk = last
            slots.append(blk * self.block_size + off)
            self._lens[sid] = n + 1
        return slots, cows

    def append_tokens(self, sid: int, count: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """``count`` tokens to one sequence (a prefill), each token one append; all-or-nothing."""
        if sid not in self._tables:
            raise KeyError(f"no sequence {sid}")
        n = self._lens[sid]
        need = 0
        if count and n % self.block_size and self._ref[self._tables[sid][-1]] > 1:
            need += 1                       # the copy of the shared, partly filled last block
        need += blocks_needed(n + count, self.block_size) - blocks_needed(n, self.block_size)
        if need > self._available():
            raise OutOfBlocks(f"{count} tokens need {need} blocks, {self._available()} available")
        slots, cows = [], []
        for _ in range(count):
            s, c = self.append(sid)
            slots.append(s)
            if c is not None:
                cows.append(c)
        return slots, cows

    def fork(self, parent: int, child: int) -> None:
        if parent not in self._tables:
            raise KeyError(f"no sequence {parent}")
        if child in self._tables:
            raise KeyError(f"sequence {child} exists")
        table = list(self._tables[parent])
        for blk in table:
            self._ref[blk] += 1
        self._tables[child] = table
        self._lens[child] = self._lens[parent]

    def free_seq(self, sid: int) -> None:
        table = self._tables.pop(sid)
        del self._lens[sid]
        for blk in reversed(table):
            self._ref[blk] -= 1
            if self._ref[blk] == 0:
                self._release(blk)

    # -- where blocks come from and go to (the prefix cache overrides these) ----
    def _available(self) -> int:
        return len(self._free)

    def _take(self) -> int:
        return self._free.pop()

    def _release(self, blk: int) -> None:
        self._free.append(blk)

    # -- queries -----------------------------------------------------------------
    def block_table(self, sid: int) -> List[int]:
        return list(self._tables[sid])

    def seq_len(self, sid: int) -> int:
        return self._lens[sid]

    def refcount(self, blk: int) -> int:
        return self._ref[blk]

    def free_list(self) -> List[int]:
        """Free blocks, next-to-pop first."""
        return list(reversed(self._free))

    def seqs(self) -> List[int]:
        return list(self._tables)

    def stats(self) -> Dict[str, float]:
        """Pool usage: free/used/shared blocks and the slot waste of the used blocks.

        A physical block's occupied slots are the most tokens any sequence
        referencing it keeps there; waste = 1 - occupied / allocated slots.
        """
        occupied: Dict[int, int] = {}
        for sid, table in self._tables.items():
            n = self._lens[sid]
            for j, blk in enumerate(table):
                fill = min(self.block_size, n - j * self.block_size)
                occupied[blk] = max(occupied.get(blk, 0), fill)
        used = sum(1 for r in self._ref if r > 0)
        shared = sum(1 for r in self._ref if r > 1)
        alloc = used * self.block_size
        occ = sum(occupied.values())
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self._free),
            "used_blocks": used,
            "shared_blocks": shared,
            "allocated_slots": alloc,
            "occupied_slots": occ,
            "waste": (1.0 - occ / alloc) if alloc else 0.0,
        }


def prereservation_waste(used_tokens: int, max_len: int) -> float:
    """Fraction of a max-length contiguous reservation left unused
    ("vLLM 核心概念", section "传统方法的痛点")."""
    return (max_len - used_tokens) / max_len


def blocks_needed(tokens: int, block_size: int = 16) -> int:
    """Blocks a sequence of ``tokens`` tokens holds under on-demand allocation."""
    return -(-tokens // block_size)
