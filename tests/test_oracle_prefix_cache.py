"""Pins of the prefix-caching oracle.

* The pages' two scenarios worked by hand: a 2000-token system prompt shared by
  three users ("vLLM 核心概念", 前缀缓存, 共享系统提示) and a multi-turn
  conversation carrying its history ("vLLM 核心概念", 前缀缓存, 多轮对话).
* Hand-worked eviction, tenant and invalidation cases.
* A content check independent of the index: a simulated pool stores, for every
  slot, the full token prefix its K/V would be computed from; after every
  operation each live sequence must find exactly its own prefixes in its
  blocks.  Reuse of a wrong block fails it whatever the index does.
* Planted mistakes (no token left to compute, key by a block's own tokens,
  evicting the newest block, evicting before the free stack is empty, tenant
  dropped from the key) each fail a pin.
"""

import random

import pytest

from oracle.prefix_cache import RefPrefixCache

BS = 16


class Driver:
    """Runs requests through a manager, keeping the simulated K/V pool and checking it."""

    def __init__(self, bm):
        self.bm = bm
        self.pool = {}            # slot -> the prefix (tuple of token ids) its K/V encodes
        self.tokens = {}          # sid -> its token ids

    def _write(self, sid, slots, cows):
        for src, dst in cows:
            for o in range(BS):
                if src * BS + o in self.pool:
                    self.pool[dst * BS + o] = self.pool[src * BS + o]
        toks = self.tokens[sid]
        start = len(toks) - len(slots)
        for i, s in enumerate(slots):
            self.pool[s] = tuple(toks[:start + i + 1])

    def request(self, sid, prompt, tenant=0):
        """Admit a prompt: reuse cached blocks, prefill the rest, commit every id."""
        cached = self.bm.add_seq_cached(sid, prompt, tenant)
        rest = list(prompt[cached:])
        try:
            slots, cows = self.bm.append_tokens(sid, len(rest))
        except Exception:                       # not admitted: give the matched blocks back
            self.bm.free_seq(sid)
            raise
        self.tokens[sid] = list(prompt)
        self._write(sid, slots, cows)
        self.bm.commit_tokens(sid, rest)
        self.check()
        return cached

    def generate(self, sid, new_tokens):
        for t in new_tokens:
            slot, cow = self.bm.append(sid)
            self.tokens[sid].append(t)
            self._write(sid, [slot], [cow] if cow else [])
            self.bm.commit_tokens(sid, [t])
        self.check()

    def fork(self, parent, child):
        self.bm.fork(parent, child)
        self.tokens[child] = list(self.tokens[parent])
        self.check()

    def free(self, sid):
        self.bm.free_seq(sid)
        del self.tokens[sid]
        self.check()

    def check(self):
        ref = {}
        for sid, toks in self.tokens.items():
            table = self.bm.block_table(sid)
            assert self.bm.seq_len(sid) == len(toks)
            for p in range(len(toks)):
                slot = table[p // BS] * BS + p % BS
                assert self.pool.get(slot) == tuple(toks[:p + 1]), (sid, p)
            for b in table:
                ref[b] = ref.get(b, 0) + 1
        for b in range(self.bm.num_blocks):
            assert self.bm.refcount(b) == ref.get(b, 0)
        free = self.bm.free_list()
        evict = self.bm.evictable_blocks()
        used = [b for b in range(self.bm.num_blocks) if ref.get(b, 0)]
        assert sorted(free + evict + used) == list(range(self.bm.num_blocks))
        assert set(evict) <= set(self.bm.cached_blocks())


def toks(seed, n, vocab=32000):
    r = random.Random(seed)
    return [r.randrange(vocab) for _ in range(n)]


# -- the pages' scenarios -------------------------------------------------------------
def test_shared_system_prompt_is_computed_once():
    system = toks(1, 2000)                      # 2000 tokens = 125 full blocks
    d = Driver(RefPrefixCache(400))
    assert d.request("A", system + toks(2, 10)) == 0
    assert d.request("B", system + toks(3, 12)) == 2000
    assert d.request("C", system + toks(4, 7)) == 2000
    st = d.bm.prefix_stats()
    assert (st["requests"], st["query_blocks"], st["hit_blocks"]) == (3, 375, 250)
    assert d.bm.block_table("B")[:125] == d.bm.block_table("A")[:125]
    assert d.bm.stats()["used_blocks"] == 128    # 125 shared + one private block each
    assert st["cached_blocks"] == 125           # the 10/12/7-token tails are not full


def test_multi_turn_history_is_reused():
    d = Driver(RefPrefixCache(64))
    turn1 = toks(5, 40)
    assert d.request(1, turn1) == 0
    answer = toks(6, 23)
    d.generate(1, answer)                       # 63 tokens: 3 full blocks
    d.free(1)
    turn2 = turn1 + answer + toks(7, 15)        # 78 tokens, 4 lookups allowed
    assert d.request(2, turn2) == 48
    assert d.bm.prefix_stats()["hit_blocks"] == 3


def test_one_prompt_token_is_always_left_to_compute():
    d = Driver(RefPrefixCache(16))
    p = toks(8, 32)
    d.request(1, p)
    d.free(1)
    assert d.request(2, p) == 16                # (32 - 1) // 16 = 1 block
    assert d.request(3, p + [5]) == 32          # 33 tokens: both blocks
    assert d.request(4, p[:16]) == 0            # (16 - 1) // 16 = 0


def test_only_whole_prefixes_match():
    a, b, c, e, f = (toks(s, 16) for s in (10, 11, 12, 13, 14))
    d = Driver(RefPrefixCache(32))
    d.request("X", a + b + [1])                 # indexes a | a+b
    d.request("W", c + f + [1])                 # indexes c | c+f
    assert d.request("Y", c + b + e + [1]) == 16     # c hits; (c, b) was never computed
    assert d.request("Z", a + e + [1]) == 16


def test_tenants_do_not_share():
    p = toks(15, 40)
    d = Driver(RefPrefixCache(32))
    d.request(1, p, tenant=7)
    assert d.request(2, p, tenant=8) == 0
    assert d.request(3, p, tenant=7) == 32


# -- eviction, hand-worked -----------------------------------------------------------
def test_lru_eviction_takes_free_blocks_first_then_the_oldest_release():
    d = Driver(RefPrefixCache(6))               # free stack pops 0, 1, 2, ...
    pa = toks(20, 33)
    d.request("A", pa)                          # blocks 0, 1 indexed; 2 partial
    assert d.bm.block_table("A") == [0, 1, 2]
    d.free("A")                                 # releases 2 (free), 1 (t=0), 0 (t=1)
    assert d.bm.free_list() == [2, 3, 4, 5]
    assert d.bm.evictable_blocks() == [1, 0]
    d.request("B", toks(21, 65))                # 5 blocks: 2, 3, 4, 5, then evicts 1
    assert d.bm.block_table("B") == [2, 3, 4, 5, 1]
    assert d.bm.prefix_stats()["evictions"] == 1
    d.free("B")
    assert d.request("C", pa) == 16             # block 0 survives, block 1 was evicted
    assert d.bm.block_table("C")[0] == 0


def test_a_hit_revives_an_evictable_block_and_renews_its_age():
    d = Driver(RefPrefixCache(8))
    p, q = toks(30, 33), toks(31, 33)
    d.request("P", p)
    d.request("Q", q)
    d.free("P")                                 # P's blocks 1, 0 released first
    d.free("Q")
    assert d.bm.evictable_blocks() == [1, 0, 4, 3]   # P: blocks 0, 1, 2; Q: 3, 4, 5
    d.request("P2", p[:17])                     # hits block 0; its own token goes to block 5
    assert d.bm.block_table("P2") == [0, 5]
    d.free("P2")                                # block 0 is now the newest release
    assert d.bm.evictable_blocks() == [1, 4, 3, 0]


def test_invalidation_drops_every_entry():
    d = Driver(RefPrefixCache(8))
    p = toks(40, 40)
    d.request(1, p)
    d.free(1)                                   # 2 free (partial block), 1 and 0 evictable
    d.bm.reset()
    assert d.bm.cached_blocks() == [] and d.bm.evictable_blocks() == []
    assert d.bm.free_list()[:3] == [0, 1, 2]    # pushed oldest first: 1, then 0 on top
    assert d.request(2, p) == 0


# -- random traces through the content check -------------------------------------------
def random_trace(seed, bm, steps=120):
    r = random.Random(seed)
    d = Driver(bm)
    # prompts made of a few recurring 16-token chunks, so equal blocks follow different
    # prefixes, plus ragged tails
    chunks = [toks(seed * 100 + i, 16) for i in range(3)]
    prompts = [sum((r.choice(chunks) for _ in range(r.randrange(1, 6))), [])
               + toks(seed * 100 + 10 + i, r.randrange(0, 20)) for i in range(6)]
    live, nid = [], 0
    for _ in range(steps):
        op = r.random()
        try:
            if op < 0.35 or not live:
                base = r.choice(prompts)
                p = base[:r.randrange(1, len(base) + 1)] + toks(r.randrange(10 ** 6), r.randrange(0, 20))
                d.request(nid, p, tenant=r.randrange(2))
                live.append(nid)
                nid += 1
            elif op < 0.6:
                d.generate(r.choice(live), toks(r.randrange(10 ** 6), r.randrange(1, 20)))
            elif op < 0.7:
                d.fork(r.choice(live), nid)
                live.append(nid)
                nid += 1
            else:
                sid = live.pop(r.randrange(len(live)))
                d.free(sid)
        except Exception as e:                  # out of blocks: the failed call changed nothing
            if type(e).__name__ != "OutOfBlocks":
                raise
            d.check()
    return d


@pytest.mark.parametrize("seed", range(12))
def test_random_traces_keep_every_sequence_content_exact(seed):
    d = random_trace(seed, RefPrefixCache(48 if seed % 2 else 200))
    st = d.bm.prefix_stats()
    assert st["hit_blocks"] <= st["query_blocks"]


def test_random_traces_do_hit_and_evict():
    hits = evictions = 0
    for seed in range(12):
        st = random_trace(seed, RefPrefixCache(48 if seed % 2 else 200)).bm.prefix_stats()
        hits += st["hit_blocks"]
        evictions += st["evictions"]
    assert hits > 100 and evictions > 20


# -- planted mistakes each fail a pin ------------------------------------------------------
class NoTokenLeft(RefPrefixCache):
    def _lookup_limit(self, n):
        return n // self.block_size


class OwnTokensKey(RefPrefixCache):
    def _key(self, tenant, prefix):
        return (tenant, tuple(prefix[-self.block_size:]))


class NoTenant(RefPrefixCache):
    def _key(self, tenant, prefix):
        return (0, tuple(prefix))


class EvictNewest(RefPrefixCache):
    def _take(self):
        if self._free:
            return self._free.pop()
        blk = max(self._evictable, key=self._evictable.get)
        del self._evictable[blk]
        del self._index[self._block_key.pop(blk)]
        self.evictions += 1
        return blk


class EvictFirst(RefPrefixCache):
    def _take(self):
        if not self._evictable:
            return self._free.pop()
        blk = min(self._evictable, key=self._evictable.get)
        del self._evictable[blk]
        del self._index[self._block_key.pop(blk)]
        self.evictions += 1
        return blk


PINS = [test_shared_system_prompt_is_computed_once, test_multi_turn_history_is_reused,
        test_one_prompt_token_is_always_left_to_compute, test_only_whole_prefixes_match,
        test_tenants_do_not_share, test_lru_eviction_takes_free_blocks_first_then_the_oldest_release,
        test_invalidation_drops_every_entry]


@pytest.mark.parametrize("cls", [NoTokenLeft, OwnTokensKey, NoTenant, EvictNewest, EvictFirst])
def test_pins_catch_planted_mistakes(monkeypatch, cls):
    failed = 0
    monkeypatch.setitem(globals(), "RefPrefixCache", cls)
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, cls.__name__


def test_own_tokens_key_breaks_the_content_check(monkeypatch):
    """Independently of the hand-worked cases, reusing a block by its own tokens hands a
    sequence K/V computed from another prefix."""
    with pytest.raises(AssertionError):
        for seed in range(12):
            random_trace(seed, OwnTokensKey(200))
