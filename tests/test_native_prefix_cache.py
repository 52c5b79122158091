"""The native prefix cache (pa_bm_* in libpa.so) against the oracle, on the CPU.

Random request traces run in lockstep through both; after every operation the
returned slots, copy-on-write pairs and cached-token counts, and the whole state
(tables, lengths, reference counts, free stack, LRU order, index, statistics)
must be identical.  The oracle's hand-worked scenarios also run on the native
manager, through the same simulated K/V content check.
"""

import random

import numpy as np
import pytest

from oracle.block_manager import OutOfBlocks as RefOutOfBlocks
from oracle.prefix_cache import RefPrefixCache
from tests import test_oracle_prefix_cache as P

N = pytest.importorskip("paged_kv_cache_385_amd._native")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    try:
        N.lib()
    except ImportError as e:
        pytest.fail(str(e))


def native(num_blocks, free_order=None):
    from paged_kv_cache_385_amd.block_manager import BlockManager
    return BlockManager(num_blocks, free_order=free_order, prefix_caching=True)


# -- the oracle's hand-worked scenarios, on the native manager -------------------------
@pytest.mark.parametrize("pin", P.PINS + [P.test_a_hit_revives_an_evictable_block_and_renews_its_age],
                         ids=lambda f: f.__name__)
def test_native_passes_the_oracle_pins(monkeypatch, pin):
    ids = {}

    class Native:
        """Native manager under the oracle's test driver (string ids mapped to ints)."""

        def __init__(self, nb):
            self.bm = native(nb)
            self.num_blocks = nb

        def __getattr__(self, name):
            fn = getattr(self.bm, name)

            def call(*a, **k):
                if a and isinstance(a[0], str):
                    a = (ids.setdefault(a[0], len(ids)),) + a[1:]
                return fn(*a, **k)
            return call

        def reset(self):
            self.bm.reset_prefix_cache()

    monkeypatch.setitem(P.__dict__, "RefPrefixCache", Native)
    pin()


# -- lockstep random traces ------------------------------------------------------------
def same_state(ref, nat, live):
    for sid in live:
        assert nat.block_table(sid) == ref.block_table(sid)
        assert nat.seq_len(sid) == ref.seq_len(sid)
    assert [nat.refcount(b) for b in range(ref.num_blocks)] == \
        [ref.refcount(b) for b in range(ref.num_blocks)]
    assert nat.free_list() == ref.free_list()
    assert nat.evictable_blocks() == ref.evictable_blocks()
    assert nat.cached_blocks() == ref.cached_blocks()
    assert nat.prefix_stats() == ref.prefix_stats()
    st_n, st_r = nat.stats(), ref.stats()
    for k in ("free_blocks", "used_blocks", "shared_blocks", "occupied_slots"):
        assert st_n[k] == st_r[k], k


def both(ref, nat, fn, *args):
    """Call fn on both; both succeed with equal results or both run out of blocks."""
    try:
        r = getattr(ref, fn)(*args)
        r_err = None
    except RefOutOfBlocks:
        r, r_err = None, True
    try:
        n = getattr(nat, fn)(*args)
        n_err = None
    except N.OutOfBlocks:
        n, n_err = None, True
    assert r_err == n_err, (fn, args)
    if r_err:
        return None
    if fn in ("append_tokens", "append_batch"):
        assert list(map(int, n[0])) == list(r[0]), fn
        assert [tuple(map(int, c)) for c in n[1]] == [tuple(c) for c in r[1]], fn
    elif fn == "append":
        assert (n[0], n[1]) == (r[0], r[1])
    else:
        assert n == r, fn
    return r


def lockstep(seed, num_blocks, steps=300):
    r = random.Random(seed)
    order = list(range(num_blocks))
    r.shuffle(order)
    ref, nat = RefPrefixCache(num_blocks, 16, order), native(num_blocks, order)
    chunks = [P.toks(seed * 7 + i, 16) for i in range(4)]
    prompts = [sum((r.choice(chunks) for _ in range(r.randrange(1, 8))), [])
               + P.toks(seed * 7 + 50 + i, r.randrange(0, 24)) for i in range(8)]
    live, nid, pending = [], 0, {}
    for _ in range(steps):
        op = r.random()
        if op < 0.3 or not live:
            base = r.choice(prompts)
            p = base[:r.randrange(1, len(base) + 1)] + P.toks(r.randrange(10 ** 6), r.randrange(0, 9))
            tenant = int(r.random() < 0.2)
            cached = both(ref, nat, "add_seq_cached", nid, p, tenant)
            if both(ref, nat, "append_tokens", nid, len(p) - cached) is None:
                both(ref, nat, "free_seq", nid)
            else:
                pending[nid] = p[cached:]
                live.append(nid)
                if r.random() < 0.7:             # most prompts commit at once
                    both(ref, nat, "commit_tokens", nid, pending[nid])
                    pending[nid] = []
            nid += 1
        elif op < 0.45:
            sid = r.choice(live)                 # commit some of what is pending
            k = r.randrange(0, len(pending[sid]) + 1)
            both(ref, nat, "commit_tokens", sid, pending[sid][:k])
            pending[sid] = pending[sid][k:]
        elif op < 0.6:
            group = r.sample(live, r.randrange(1, min(len(live), 6) + 1))
            toks = [r.randrange(40) for _ in group]          # a tiny vocabulary: repeats
            if both(ref, nat, "append_batch", group) is not None:
                for sid, t in zip(group, toks):
                    pending[sid].append(t)
                ready = [s for s in group if len(pending[s]) == 1]
                if ready:
                    both(ref, nat, "commit_batch", ready, [pending[s][0] for s in ready])
                    for s in ready:
                        pending[s] = []
        elif op < 0.68:
            parent = r.choice(live)
            both(ref, nat, "fork", parent, nid)
            pending[nid] = list(pending[parent])
            live.append(nid)
            nid += 1
        elif op < 0.685:
            ref.reset()
            nat.reset_prefix_cache()
        else:
            sid = live.pop(r.randrange(len(live)))
            both(ref, nat, "free_seq", sid)
            del pending[sid]
        same_state(ref, nat, live)
    return ref.prefix_stats()


@pytest.mark.parametrize("seed", range(10))
def test_lockstep_with_the_oracle(seed):
    st = lockstep(seed, 40 if seed % 2 else 160)
    assert st["requests"] > 0


def test_lockstep_traces_exercise_hits_evictions_and_resets():
    hits = evictions = 0
    for seed in range(10):
        st = lockstep(seed, 40 if seed % 2 else 160)
        hits += st["hit_blocks"]
        evictions += st["evictions"]
    assert hits > 500 and evictions > 60


# -- errors --------------------------------------------------------------------------------
def test_prefix_calls_need_prefix_caching_on():
    from paged_kv_cache_385_amd.block_manager import BlockManager
    bm = BlockManager(8)
    with pytest.raises(N.PaError) as e:
        bm.add_seq_cached(1, [1, 2, 3])
    assert e.value.status == N.PA_ERR_UNSUPPORTED
    bm.add_seq(1)
    bm.append_tokens(1, 3)
    with pytest.raises(N.PaError) as e:
        bm.commit_tokens(1, [1, 2, 3])
    assert e.value.status == N.PA_ERR_UNSUPPORTED
    # turning it on needs an empty manager
    with pytest.raises(N.PaError) as e:
        N.check(bm._lib.pa_bm_enable_prefix_cache(bm._h), "pa_bm_enable_prefix_cache")
    assert e.value.status == N.PA_ERR_INVALID_ARG
    assert bm.prefix_stats()["requests"] == 0


def test_commit_validation_changes_nothing():
    bm = native(8)
    assert bm.add_seq_cached(1, list(range(20))) == 0
    bm.append_tokens(1, 20)
    with pytest.raises(N.PaError):
        bm.commit_tokens(1, list(range(21)))           # more ids than slots
    bm.commit_tokens(1, list(range(15)))
    assert bm.cached_blocks() == []
    bm.add_seq(2)
    with pytest.raises(N.PaError):
        bm.commit_batch([1, 2], [15, 0])              # sequence 2 has nothing to commit
    with pytest.raises(N.PaError):
        bm.commit_batch([1, 1], [15, 16])              # twice the same sequence
    bm.commit_batch([1], [15])
    assert bm.cached_blocks() == [0]
    with pytest.raises(N.PaError):
        bm.add_seq_cached(3, [1], tenant=-1)
    with pytest.raises(N.PaError):
        bm.add_seq_cached(1, [1])                      # exists


def test_hundred_thousand_block_lookups_are_fast():
    """A 2000-token shared system prompt, 400 requests: lookups stay in the microseconds."""
    import time
    bm = native(40000)
    system = P.toks(1, 2000)
    t0 = time.perf_counter()
    for i in range(400):
        p = system + P.toks(1000 + i, 30)
        c = bm.add_seq_cached(i, p)
        bm.append_tokens(i, len(p) - c)
        bm.commit_tokens(i, p[c:])
    dt = time.perf_counter() - t0
    st = bm.prefix_stats()
    assert st["hit_blocks"] == 399 * 125 and st["query_blocks"] == 400 * 126
    assert dt < 5.0


# -- batched admission -------------------------------------------------------------------
def oracle_admit(ref, sids, prompts, tenants):
    """The oracle's admission of a batch, request by request (match, append, commit); stops
    at the first request that does not fit, releasing its matched blocks."""
    cached, slots = [], []
    for sid, p, t in zip(sids, prompts, tenants):
        c = ref.add_seq_cached(sid, p, t)
        try:
            sl, cows = ref.append_tokens(sid, len(p) - c)
        except RefOutOfBlocks:
            ref.free_seq(sid)
            return cached, slots, len(cached)
        assert not cows
        ref.commit_tokens(sid, p[c:])
        cached.append(c)
        slots += sl
    return cached, slots, len(cached)


@pytest.mark.parametrize("seed", range(6))
def test_admit_batch_matches_request_by_request_admission(seed):
    r = random.Random(seed)
    nb = 24 if seed % 2 else 300
    order = list(range(nb))
    r.shuffle(order)
    ref, nat = RefPrefixCache(nb, 16, order), native(nb, order)
    chunks = [P.toks(seed * 13 + i, 16) for i in range(3)]
    live, nid, ran_out = [], 0, 0
    for _ in range(40):
        k = r.randrange(0, 9)
        prompts = [sum((r.choice(chunks) for _ in range(r.randrange(0, 6))), [])
                   + P.toks(r.randrange(10 ** 6), r.randrange(1, 30)) for _ in range(k)]
        tenants = [int(r.random() < 0.25) for _ in range(k)]
        sids = list(range(nid, nid + k))
        nid += k
        want_c, want_s, want_k = oracle_admit(ref, sids, prompts, tenants)
        flat = np.array([t for p in prompts for t in p], dtype=np.int32)
        offs = np.concatenate([[0], np.cumsum([len(p) for p in prompts])]).astype(np.int64)
        try:
            c, sl, got_k = nat.admit_batch(sids, flat, offs, tenants)
        except N.OutOfBlocks as e:
            got_k = e.admitted
            ran_out += 1
            assert want_k < k
        else:
            assert list(c) == want_c and list(map(int, sl)) == want_s
        assert got_k == want_k
        live += sids[:got_k]
        same_state(ref, nat, live)
        for sid in r.sample(live, r.randrange(0, len(live) + 1)):
            live.remove(sid)
            ref.free_seq(sid)
            nat.free_seq(sid)
        same_state(ref, nat, live)
    if seed % 2:
        assert ran_out > 0
    assert nat.prefix_stats()["hit_blocks"] > 0


def test_admit_batch_validates_before_changing_anything():
    bm = native(16)
    flat = np.arange(40, dtype=np.int32)
    with pytest.raises(N.PaError):
        bm.admit_batch([1, 1], flat, [0, 20, 40])          # twice the same sequence
    with pytest.raises(N.PaError):
        bm.admit_batch([1, 2], flat, [0, 30, 20])          # offsets go back
    with pytest.raises(N.PaError):
        bm.admit_batch([1, 2], flat, [0, 20, 40], tenants=[0, -3])
    assert bm.prefix_stats()["requests"] == 0 and bm.free_list() == list(range(16))
    c, sl, k = bm.admit_batch([1, 2], flat, [0, 20, 40])
    assert (list(c), k, len(sl)) == ([0, 0], 2, 40)
