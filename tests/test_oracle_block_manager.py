"""Pins of the reference block manager: the pages' worked examples and invariants."""

import json
import os

import numpy as np
import pytest

from oracle import block_manager as BM
from oracle import cache as C
from tests.conftest import GOLDEN
from workloads import make_workload


def _order_starting(prefix, n):
    rest = [b for b in range(n) if b not in prefix]
    return list(prefix) + rest


def test_block_table_example_and_growth():
    g = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    bm = BM.RefBlockManager(16, g["block_size"], _order_starting(g["block_table"], 16))
    bm.add_seq(0)
    states = {st["after_tokens"]: st for st in g["growth"]}
    slots = []
    for t in range(g["tokens"]):
        if t in states:
            assert bm.block_table(0) == states[t]["table"]
        s, cow = bm.append(0)
        assert cow is None
        slots.append(s)
        if t in states and "next_allocates" in states[t]:
            assert bm.block_table(0)[-1] == states[t]["next_allocates"]
    assert bm.block_table(0) == g["block_table"]
    for lo, hi, blk in g["token_ranges"]:
        for t in range(lo, hi + 1):
            assert slots[t] // 16 == blk and slots[t] % 16 == t - lo


def test_hundred_tokens_take_seven_blocks():
    g = json.load(open(os.path.join(GOLDEN, "hundred_tokens.json")))
    bm = BM.RefBlockManager(32, g["block_size"])
    bm.add_seq(1)
    bm.append_tokens(1, g["tokens"])
    assert len(bm.block_table(1)) == g["blocks"]
    assert BM.blocks_needed(g["tokens"]) == g["blocks"]
    st = bm.stats()
    assert st["used_blocks"] == g["blocks"]
    assert st["occupied_slots"] == g["full_blocks"] * 16 + g["tokens_in_last_block"]
    assert st["allocated_slots"] - st["occupied_slots"] == 16 - g["tokens_in_last_block"]


def test_prereservation_waste_golden():
    g = json.load(open(os.path.join(GOLDEN, "prereservation_waste.json")))
    for case in g["cases"]:
        w = BM.prereservation_waste(case["used_tokens"], g["max_len"]) * 100
        assert case["used_tokens"] + case["reserved_unused"] == g["max_len"]
        # the page truncates to at most one decimal
        assert case["printed_waste_percent"] <= w < case["printed_waste_percent"] + 0.7


def test_paged_waste_is_confined_to_last_block():
    rng = np.random.default_rng(0)
    bm = BM.RefBlockManager(400, 16, rng.permutation(400))
    lens = rng.integers(1, 300, size=20)
    for i, n in enumerate(lens):
        bm.add_seq(i)
        bm.append_tokens(i, int(n))
    st = bm.stats()
    assert st["allocated_slots"] - st["occupied_slots"] <= 15 * len(lens)
    assert st["occupied_slots"] == int(lens.sum())


def test_fork_shares_and_cow_only_on_divergence():
    bm = BM.RefBlockManager(64, 16, list(range(64)))
    bm.add_seq(0)
    bm.append_tokens(0, 40)                 # blocks 0,1 full, block 2 holds 8 tokens
    for c in (1, 2, 3):
        bm.fork(0, c)
    assert [bm.refcount(b) for b in (0, 1, 2)] == [4, 4, 4]
    # first divergent write of sequences 0..2 copies the shared partial block
    cows = []
    for sid in (0, 1, 2):
        s, cow = bm.append(sid)
        cows.append(cow)
        assert s % 16 == 8
    assert [c[0] for c in cows] == [2, 2, 2]
    assert len({c[1] for c in cows}) == 3
    assert bm.refcount(2) == 1
    # the last sharer writes in place
    s, cow = bm.append(3)
    assert cow is None and s == 2 * 16 + 8
    # full shared blocks are never copied
    assert [bm.refcount(b) for b in (0, 1)] == [4, 4]


def test_fork_at_block_boundary_never_copies():
    bm = BM.RefBlockManager(32, 16)
    bm.add_seq(0)
    bm.append_tokens(0, 32)
    bm.fork(0, 1)
    _, c0 = bm.append(0)
    _, c1 = bm.append(1)
    assert c0 is None and c1 is None
    assert bm.block_table(0)[:2] == bm.block_table(1)[:2]
    assert bm.block_table(0)[2] != bm.block_table(1)[2]


def test_shared_prefix_workload_cow_counts():
    wl = make_workload(4)
    bm = BM.RefBlockManager(wl.num_blocks, 16, wl.free_order)
    cows = []
    for op in wl.setup:
        if op[0] == "add":
            bm.add_seq(op[1])
        elif op[0] == "fork":
            bm.fork(op[1], op[2])
        else:
            cows += bm.append_tokens(op[1], op[4])[1]
    _, step_cows = bm.append_batch([op[1] for op in wl.step])
    cows += step_cows
    assert len(cows) == 7 * 16       # 7 copies per prompt, the 8th sharer writes in place
    # literal block-aligned prefix: nothing to copy
    wl0 = make_workload(4, extra_max=0)
    bm0 = BM.RefBlockManager(wl0.num_blocks, 16, wl0.free_order)
    n = 0
    for op in wl0.setup:
        if op[0] == "add":
            bm0.add_seq(op[1])
        elif op[0] == "fork":
            bm0.fork(op[1], op[2])
        else:
            n += len(bm0.append_tokens(op[1], op[4])[1])
    n += len(bm0.append_batch([op[1] for op in wl0.step])[1])
    assert n == 0


def _snapshot(bm):
    return (bm.free_list(), {s: (bm.block_table(s), bm.seq_len(s)) for s in bm.seqs()},
            [bm.refcount(b) for b in range(bm.num_blocks)])


def test_exhaustion_is_atomic():
    bm = BM.RefBlockManager(4, 16)
    bm.add_seq(0)
    bm.append_tokens(0, 48)          # 3 blocks
    bm.add_seq(1)
    bm.append_tokens(1, 16)          # 4th block
    snap = _snapshot(bm)
    with pytest.raises(BM.OutOfBlocks):
        bm.append(0)
    assert _snapshot(bm) == snap
    bm.fork(1, 2)
    bm.free_seq(1)
    snap = _snapshot(bm)
    with pytest.raises(BM.OutOfBlocks):
        bm.append_batch([2, 0])
    assert _snapshot(bm) == snap


def test_prefill_append_counts_the_copy_on_write_block():
    """append_tokens is all or nothing, and its block count includes the private copy of
    a shared, partly filled last block.  Worked by hand on a 6-block pool (free order
    0, 1, ..., so blocks are taken in ascending order):
      seq 0 holds 20 tokens in blocks [0, 1] (block 1 holds 4); seq 1 is its fork, so
      both blocks have two references and blocks 2..5 are free.
      61 more tokens for seq 1 reach 81 tokens = 6 blocks: the copy of block 1 plus 4
      new blocks = 5 > 4 free -> refused, nothing changes.  (A count that leaves out
      the copy would see 4 <= 4, start, and fail on token 81 with the pool changed.)
      60 tokens reach 80 = 5 blocks: copy + 3 new = 4 -> accepted.  Block 1 is copied
      to 2 (pair (1, 2)), positions 20..31 land in block 2, then 32..47 in 3, 48..63
      in 4 and 64..79 in 5.
      seq 0 is now block 1's only holder and fills it in place (12 tokens, no block);
      its 33rd token needs a block the empty pool does not have -> refused."""
    bm = BM.RefBlockManager(6, 16)
    bm.add_seq(0)
    assert bm.append_tokens(0, 20) == (list(range(0, 20)), [])
    bm.fork(0, 1)
    snap = _snapshot(bm)
    with pytest.raises(BM.OutOfBlocks):
        bm.append_tokens(1, 61)
    assert _snapshot(bm) == snap
    slots, cows = bm.append_tokens(1, 60)
    assert cows == [(1, 2)]
    assert slots == (list(range(2 * 16 + 4, 3 * 16)) + list(range(3 * 16, 6 * 16)))
    assert bm.block_table(1) == [0, 2, 3, 4, 5]
    assert bm.block_table(0) == [0, 1]
    assert [bm.refcount(b) for b in range(6)] == [2, 1, 1, 1, 1, 1]
    assert bm.free_list() == []
    assert bm.append_tokens(0, 12) == (list(range(16 + 4, 32)), [])
    snap = _snapshot(bm)
    with pytest.raises(BM.OutOfBlocks):
        bm.append_tokens(0, 1)
    assert _snapshot(bm) == snap


def test_free_returns_blocks_first_logical_on_top():
    bm = BM.RefBlockManager(8, 16, [3, 1, 4, 0, 5, 2, 6, 7])
    bm.add_seq(0)
    bm.append_tokens(0, 40)
    assert bm.block_table(0) == [3, 1, 4]
    bm.free_seq(0)
    assert bm.free_list()[:3] == [3, 1, 4]
    bm.add_seq(1)
    bm.append_tokens(1, 33)
    assert bm.block_table(1) == [3, 1, 4]


@pytest.mark.parametrize("seed", range(8))
def test_invariants_on_random_traces(seed):
    rng = np.random.default_rng(seed)
    nb = 96
    bm = BM.RefBlockManager(nb, 16, rng.permutation(nb))
    live, next_id = [], 0
    for _ in range(600):
        r = rng.random()
        try:
            if r < 0.15 or not live:
                bm.add_seq(next_id)
                live.append(next_id)
                next_id += 1
            elif r < 0.25:
                p = live[int(rng.integers(len(live)))]
                bm.fork(p, next_id)
                live.append(next_id)
                next_id += 1
            elif r < 0.32:
                s = live.pop(int(rng.integers(len(live))))
                bm.free_seq(s)
            else:
                k = int(rng.integers(1, min(len(live), 6) + 1))
                bm.append_batch(rng.choice(live, size=k, replace=False).tolist())
        except BM.OutOfBlocks:
            s = live.pop(0)
            bm.free_seq(s)
        refs = np.zeros(nb, dtype=int)
        for s in live:
            for b in bm.block_table(s):
                refs[b] += 1
            assert len(bm.block_table(s)) == BM.blocks_needed(bm.seq_len(s))
        assert refs.tolist() == [bm.refcount(b) for b in range(nb)]
        free = bm.free_list()
        assert len(set(free)) == len(free)
        assert set(free).isdisjoint({b for b in range(nb) if refs[b] > 0})
        assert len(free) + int((refs > 0).sum()) == nb


@pytest.mark.parametrize("cfg", [1, 4])
def test_trace_builds_each_sequence_exactly(cfg):
    """CPU model of the whole path: block-manager slots drive the oracle cache
    write, and every sequence read back through its table equals its logical K/V."""
    wl = make_workload(cfg)
    bm = BM.RefBlockManager(wl.num_blocks, 16, wl.free_order)
    kp, vp = C.empty_pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, fill=0x7E00)
    segs = {}

    def seg(sid):
        if sid not in segs:
            segs[sid] = wl.segment_kv(sid)
        return segs[sid]

    pending_cow = []
    writes = []
    for op in wl.setup + wl.step:
        if op[0] == "add":
            bm.add_seq(op[1])
        elif op[0] == "fork":
            bm.fork(op[1], op[2])
        else:
            _, sid, sg, start, n = op
            slots, cows = bm.append_tokens(sid, n)
            pending_cow += cows
            k, v = seg(sg)
            writes.append((k[start:start + n], v[start:start + n], slots))
    # device order: prefixes first, then every copy-on-write copy, then the rest
    first = []
    if cfg == 4:
        n_prefix = wl.notes["prompts"]
        first, rest = writes[:n_prefix], writes[n_prefix:]
    else:
        rest = writes
    for k, v, s in first:
        C.cache_write(kp, vp, k, v, s, inplace=True)
    C.copy_blocks(kp, vp, pending_cow, inplace=True)
    for k, v, s in rest:
        C.cache_write(kp, vp, k, v, s, inplace=True)
    for b in range(wl.num_seqs):
        k, v = wl.seq_kv(b, segs)
        gk, gv = C.gather_sequence(kp, vp, bm.block_table(b), int(wl.ctx_lens[b]))
        assert np.array_equal(gk, C.bits16(k)) and np.array_equal(gv, C.bits16(v)), b
