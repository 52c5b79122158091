"""Automatic prefix caching on the device: requests that reuse cached blocks compute
only their new tokens, and their attention (pa_chunk_attention over reused plus new
blocks, then pa_decode steps on blocks shared by several sequences) matches the
oracle's attention over K/V computed from scratch for the whole prompt.

K/V are prefix-dependent (workloads.prefix): a block reused after a different
prefix would hold different values and fail.  The oracle's prefix cache runs in
lockstep and fixes the expected cached-token counts and block tables.
Tolerance: 2e-3 (float16) / 1e-2 (bfloat16), max absolute error.
"""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle.prefix_cache import RefPrefixCache
from tests.gpu_harness import POISON, check_close, say
from workloads.prefix import prompt_ids, queries, system_prompt_requests, token_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import paged_kv_cache_385_amd._native as N
    N.lib()


class Scenario:
    """A device cache with prefix caching and the oracle's manager in lockstep."""

    def __init__(self, num_blocks, H, Hkv, D, dtype, seed):
        from paged_kv_cache_385_amd import PagedKVCache
        self.H, self.Hkv, self.D, self.dtype, self.seed = H, Hkv, D, dtype, seed
        self.scale = D ** -0.5
        self.cache = PagedKVCache(num_blocks, Hkv, D, dtype, "cuda", fill_bits=POISON[dtype],
                                  prefix_caching=True)
        self.ref = RefPrefixCache(num_blocks)
        self.ids = {}

    def kv(self, ids, start, n):
        return token_kv(self.seed, ids, start, n, self.Hkv, self.D, self.dtype)

    def admit(self, sid, prompt):
        cached = self.cache.admit(sid, prompt, lambda s, n: self.kv(prompt, s, n))
        want = self.ref.add_seq_cached(sid, prompt)
        self.ref.append_tokens(sid, len(prompt) - want)
        self.ref.commit_tokens(sid, prompt[want:])
        assert cached == want
        assert self.cache.bm.block_table(sid) == self.ref.block_table(sid)
        self.ids[sid] = list(prompt)
        return cached

    def prefill_attention(self, sid, cached):
        """pa_chunk_attention for the tokens the request computed itself."""
        from paged_kv_cache_385_amd import chunk_attention
        ids = self.ids[sid]
        n = len(ids) - cached
        q = queries(self.seed, sid, n, self.H, self.D, self.dtype)
        mb = -(-len(ids) // 16)
        tables, ctx, mc = self.cache.tables([sid], mb)
        starts = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        out = chunk_attention(self.cache.k_cache, self.cache.v_cache, q.cuda(), starts, tables,
                              ctx, n, mc, self.scale)
        torch.cuda.synchronize()
        k, v = self.kv(ids, 0, len(ids))
        return out, OA.chunk_attention(q, k, v, self.scale)

    def decode_step(self, sids, step):
        """One decode step of every sequence through DecodeBatch, then the ids' commit."""
        from paged_kv_cache_385_amd import DecodeBatch
        toks = [int(prompt_ids(self.seed, 10_000 + step, len(sids))[i]) for i in range(len(sids))]
        for sid, t in zip(sids, toks):
            self.ids[sid].append(t)
        kv = [self.kv(self.ids[s], len(self.ids[s]) - 1, 1) for s in sids]
        k_new = torch.cat([a for a, _ in kv]).cuda()
        v_new = torch.cat([b for _, b in kv]).cuda()
        q = queries(self.seed, 50_000 + step, len(sids), self.H, self.D, self.dtype)
        mb = max(-(-len(self.ids[s]) // 16) for s in sids)
        batch = DecodeBatch(self.cache, sids, self.H, self.scale, mb)
        out = batch.step(k_new, v_new, q.view(len(sids), self.H, self.D).cuda())
        torch.cuda.synchronize()
        self.cache.bm.commit_batch(sids, toks)
        self.ref.append_batch(sids)
        self.ref.commit_batch(sids, toks)
        ref = np.stack([OA.decode_attention(q[i], *self.kv(self.ids[s], 0, len(self.ids[s])),
                                            self.scale) for i, s in enumerate(sids)])
        return out, ref


def test_shared_system_prompt():
    """Four requests on one 2000-token system prompt (GQA-8, bf16): the first computes
    everything, the others reuse its 125 blocks; then two decode steps on the shared
    blocks."""
    sc = Scenario(600, 16, 2, 128, torch.bfloat16, seed=31)
    prompts = system_prompt_requests(31, 4, 2000, (1, 64))
    for sid, p in enumerate(prompts):
        cached = sc.admit(sid, p)
        say(f"request {sid}: {len(p)} tokens, {cached} reused")
        assert cached == (0 if sid == 0 else 2000)
        out, ref = sc.prefill_attention(sid, cached)
        rows = None if sid else np.r_[0:64, 1000:1064, len(p) - 64:len(p)]
        check_close(out, ref, sc.dtype, rows=rows, label=f"prefill of request {sid}")
    assert all(sc.cache.bm.refcount(b) == 4 for b in sc.cache.bm.block_table(0)[:125])
    for step in range(2):
        out, ref = sc.decode_step([0, 1, 2, 3], step)
        check_close(out, ref, sc.dtype, label=f"decode step {step} on shared blocks")
    st = sc.cache.bm.prefix_stats()
    assert st == sc.ref.prefix_stats()
    say(f"prefix stats: {st}")


def test_multi_turn_with_eviction():
    """A conversation's second turn reuses its first turn's blocks; unrelated requests in
    between evict part of them (a 64-block pool), so the turn reuses fewer blocks and
    recomputes the rest into blocks that held other sequences' K/V."""
    sc = Scenario(64, 8, 8, 64, torch.float16, seed=32)
    turn1 = prompt_ids(32, 1, 300)
    sc.admit(100, turn1)
    for step in range(3):
        out, ref = sc.decode_step([100], step)
        check_close(out, ref, sc.dtype, label=f"turn 1 decode {step}")
    history = list(sc.ids[100])
    sc.cache.bm.free_seq(100)
    sc.ref.free_seq(100)
    # other users take most of the pool: LRU evicts the tail of the conversation first
    for i in range(3):
        sc.admit(200 + i, prompt_ids(32, 10 + i, 250))
    for i in range(3):
        sc.cache.bm.free_seq(200 + i)
        sc.ref.free_seq(200 + i)
    turn2 = history + prompt_ids(32, 2, 41)
    cached = sc.admit(101, turn2)
    say(f"turn 2: {len(turn2)} tokens, {cached} reused, "
        f"{sc.cache.bm.prefix_stats()['evictions']} evictions so far")
    assert 0 < cached < 16 * (len(history) // 16)
    out, ref = sc.prefill_attention(101, cached)
    check_close(out, ref, sc.dtype, label="turn 2 prefill after evictions")
    assert sc.cache.bm.prefix_stats() == sc.ref.prefix_stats()


def test_tenants_and_reset_on_device():
    """The same prompt under another tenant, and after an invalidation, is recomputed in
    full; both still match the oracle."""
    sc = Scenario(128, 4, 4, 64, torch.float16, seed=33)
    p = prompt_ids(33, 1, 200)
    sc.admit(1, p)
    sc.cache.bm.free_seq(1)
    sc.ref.free_seq(1)
    cached = sc.cache.admit(2, p, lambda s, n: sc.kv(p, s, n), tenant=5)
    assert cached == 0
    sc.cache.bm.free_seq(2)
    sc.cache.bm.reset_prefix_cache()
    assert sc.ref.add_seq_cached(2, p, 5) == 0
    sc.ref.append_tokens(2, len(p))
    sc.ref.commit_tokens(2, p)
    sc.ref.free_seq(2)
    sc.ref.reset()
    assert sc.admit(3, p) == 0
    out, ref = sc.prefill_attention(3, 0)
    check_close(out, ref, sc.dtype, label="after reset")
    assert sc.cache.bm.prefix_stats() == sc.ref.prefix_stats()
