"""Pins of the swap oracle.

* Content check independent of the bookkeeping: a simulated device pool and
  host pool hold, per slot, the token prefix its K/V encode; swap pairs are
  applied as block copies; after every operation each resident sequence finds
  its own prefixes in its device blocks, and each swapped-out one in its host
  blocks.  A lost copy, a wrong pair or a reused-too-early block fails it.
* Hand-worked cases: block order, sharing kept across a swap, all-or-nothing.
* Planted mistakes (sharing not kept, pairs reversed, device blocks released
  before the copy list is made) each fail a pin.
"""

import random

import pytest

from oracle.block_manager import OutOfBlocks
from oracle.swap import RefSwapManager

BS = 16


class Driver:
    def __init__(self, bm):
        self.bm = bm
        self.dev = {}       # device slot -> prefix tuple
        self.host = {}      # host slot -> prefix tuple
        self.tokens = {}

    def _copy(self, src, dst, s_blk, d_blk):
        for o in range(BS):
            if s_blk * BS + o in src:
                dst[d_blk * BS + o] = src[s_blk * BS + o]
            else:
                dst.pop(d_blk * BS + o, None)

    def add(self, sid, n, start=0):
        self.bm.add_seq(sid)
        self.tokens[sid] = []
        try:
            self.grow(sid, n, start)
        except OutOfBlocks:
            self.bm.free_seq(sid)
            del self.tokens[sid]
            raise

    def grow(self, sid, n, start=0):
        slots, cows = self.bm.append_tokens(sid, n)
        for s, d in cows:
            self._copy(self.dev, self.dev, s, d)
        t = self.tokens[sid]
        for i, slot in enumerate(slots):
            t.append(start + len(t) + 1000 * sid)
            self.dev[slot] = tuple(t)
        self.check()

    def fork(self, parent, child):
        self.bm.fork(parent, child)
        self.tokens[child] = list(self.tokens[parent])
        self.check()

    def swap_out(self, sids):
        pairs = self.bm.swap_out(sids)
        for d, h in pairs:
            self._copy(self.dev, self.host, d, h)
        self.check()
        return pairs

    def swap_in(self, sids):
        pairs = self.bm.swap_in(sids)
        for h, d in pairs:
            self._copy(self.host, self.dev, h, d)
        self.check()
        return pairs

    def free(self, sid):
        self.bm.free_seq(sid)
        del self.tokens[sid]
        self.check()

    def check(self):
        for sid, toks in self.tokens.items():
            if self.bm.is_swapped(sid):
                table, pool = self.bm.host_table(sid), self.host
            else:
                table, pool = self.bm.block_table(sid), self.dev
            assert len(table) == -(-len(toks) // BS)
            for p in range(len(toks)):
                assert pool.get(table[p // BS] * BS + p % BS) == tuple(toks[:p + 1]), (sid, p)
        href = {}
        for sid in self.tokens:
            if self.bm.is_swapped(sid):
                for h in self.bm.host_table(sid):
                    href[h] = href.get(h, 0) + 1
        for h in range(self.bm.num_host_blocks):
            assert self.bm.host_refcount(h) == href.get(h, 0)
        free = self.bm.host_free_list()
        assert sorted(free + list(href)) == list(range(self.bm.num_host_blocks))


def test_round_trip_keeps_contents_and_sharing():
    d = Driver(RefSwapManager(16, 8))
    d.add(1, 40)                     # blocks 0, 1, 2 (2 partial)
    d.fork(1, 2)                     # shares all three
    d.grow(2, 1)                     # copy-on-write of block 2 -> 3
    assert d.bm.block_table(2) == [0, 1, 3]
    pairs = d.swap_out([1, 2])       # distinct blocks 0, 1, 2, 3 -> host 0, 1, 2, 3
    assert pairs == [(0, 0), (1, 1), (2, 2), (3, 3)]
    assert d.bm.host_table(1) == [0, 1, 2] and d.bm.host_table(2) == [0, 1, 3]
    assert d.bm.host_refcount(0) == 2 and d.bm.host_refcount(3) == 1
    # device blocks released: seq 1 last-first (2; 1 and 0 still held by 2), then seq 2 (3, 1, 0)
    assert d.bm.free_list()[:4] == [0, 1, 3, 2]
    d.add(3, 64)                     # reuses the freed device blocks
    assert d.bm.block_table(3) == [0, 1, 3, 2]
    pairs = d.swap_in([2, 1])        # seq 2 first: host 0, 1, 3, then 2
    assert [h for h, _ in pairs] == [0, 1, 3, 2]
    assert d.bm.block_table(2)[:2] == d.bm.block_table(1)[:2]     # still shared
    assert d.bm.refcount(d.bm.block_table(1)[0]) == 2
    assert d.bm.host_free_list()[:4] == [0, 1, 2, 3]


def test_a_block_shared_with_a_resident_sequence_keeps_its_device_copy():
    d = Driver(RefSwapManager(8, 8))
    d.add(1, 32)
    d.fork(1, 2)
    d.swap_out([1])
    assert d.bm.refcount(0) == 1 and d.bm.refcount(1) == 1      # still held by sequence 2
    d.grow(2, 5)
    d.swap_in([1])
    assert d.bm.block_table(1) != d.bm.block_table(2)[:2]       # separate copies now


def test_all_or_nothing():
    d = Driver(RefSwapManager(8, 2))
    d.add(1, 40)                                     # 3 blocks > 2 host blocks
    with pytest.raises(OutOfBlocks):
        d.swap_out([1])
    assert not d.bm.is_swapped(1) and d.bm.host_free_list() == [0, 1]
    d.add(2, 20)
    d.swap_out([2])
    d.add(3, 16 * 5)                                 # takes the 5 device blocks left
    with pytest.raises(OutOfBlocks):
        d.swap_in([2])
    assert d.bm.is_swapped(2)
    d.free(3)
    d.swap_in([2])
    with pytest.raises(KeyError):
        d.bm.swap_in([2])                            # not swapped out any more
    with pytest.raises(ValueError):
        d.bm.swap_out([1, 1])


def test_a_swapped_sequence_cannot_grow_but_can_end():
    d = Driver(RefSwapManager(8, 8))
    d.add(1, 20)
    d.swap_out([1])
    with pytest.raises(KeyError):
        d.bm.append(1)
    with pytest.raises(KeyError):
        d.bm.fork(1, 2)
    d.free(1)
    assert d.bm.host_free_list() == list(range(8))


def random_trace(seed, bm, steps=200):
    r = random.Random(seed)
    d = Driver(bm)
    nid = 0
    for _ in range(steps):
        resident = [s for s in d.tokens if not bm.is_swapped(s)]
        swapped = [s for s in d.tokens if bm.is_swapped(s)]
        op = r.random()
        try:
            if op < 0.25 or not d.tokens:
                nid += 1
                d.add(nid, r.randrange(1, 60))
            elif op < 0.45 and resident:
                d.grow(r.choice(resident), r.randrange(1, 20))
            elif op < 0.55 and resident:
                nid += 1
                d.fork(r.choice(resident), nid)
            elif op < 0.7 and resident:
                d.swap_out(r.sample(resident, r.randrange(1, min(3, len(resident)) + 1)))
            elif op < 0.85 and swapped:
                d.swap_in(r.sample(swapped, r.randrange(1, min(3, len(swapped)) + 1)))
            else:
                d.free(r.choice(list(d.tokens)))
        except OutOfBlocks:
            d.check()
    return d


@pytest.mark.parametrize("seed", range(10))
def test_random_traces_keep_every_sequence_intact(seed):
    random_trace(seed, RefSwapManager(24 if seed % 2 else 64, 16 if seed % 2 else 64))


# -- planted mistakes -----------------------------------------------------------------
class NoSharing(RefSwapManager):
    @staticmethod
    def _distinct(tables):
        return [b for t in tables for b in t]     # one host block per reference


class ReversedPairs(RefSwapManager):
    def swap_in(self, sids):
        return [(d, h) for h, d in super().swap_in(sids)]


class ReleaseFirst(RefSwapManager):
    """Releases the device blocks before planning the copies: swapping two sequences
    that share a block then lists that block twice, and the host tier runs short."""
    def swap_out(self, sids):
        pairs = []
        for sid in sids:
            pairs += super().swap_out([sid])
        return pairs


@pytest.mark.parametrize("cls", [NoSharing, ReversedPairs, ReleaseFirst])
def test_pins_catch_planted_mistakes(monkeypatch, cls):
    failed = 0
    monkeypatch.setitem(globals(), "RefSwapManager", cls)
    for pin in (test_round_trip_keeps_contents_and_sharing,
                test_a_block_shared_with_a_resident_sequence_keeps_its_device_copy):
        try:
            pin()
        except (AssertionError, KeyError, IndexError):
            failed += 1
    try:
        for seed in range(4):
            random_trace(seed, cls(24, 16))
    except (AssertionError, KeyError, IndexError):
        failed += 1
    assert failed > 0, cls.__name__
