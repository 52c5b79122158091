"""The seeded generators: determinism and the shapes of the five workloads."""

import numpy as np
import pytest
import torch

from workloads import CONFIG_IDS, custom_workload, make_workload


@pytest.mark.parametrize("cfg", CONFIG_IDS)
def test_shapes_and_ranges(cfg):
    wl = make_workload(cfg)
    B = wl.num_seqs
    assert wl.ctx_lens.shape == (B,)
    assert sorted(wl.free_order.tolist()) == list(range(wl.num_blocks))
    assert wl.num_heads % wl.num_kv_heads == 0
    assert wl.scale == pytest.approx(1.0 / np.sqrt(wl.head_dim))
    assert len(wl.step) == B and [op[1] for op in wl.step] == list(range(B))
    for b in range(B):
        assert sum(n for _, _, n in wl.seq_slices[b]) == wl.ctx_lens[b]
    c = wl.ctx_lens
    if cfg == 1:
        assert c.tolist() == [17, 33, 64, 100] and wl.num_blocks == 64
        assert (wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.dtype) == (8, 8, 64, torch.float16)
    elif cfg == 2:
        assert B == 64 and c.min() >= 128 and c.max() <= 2048
        assert (wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.dtype) == (32, 32, 128, torch.float16)
    elif cfg == 3:
        assert B == 128 and c.min() >= 16 and c.max() <= 4096
        assert 700 < np.median(c) < 1400
        assert (wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.dtype) == (64, 8, 128, torch.bfloat16)
    elif cfg == 4:
        assert B == 128
        pre = np.repeat(wl.notes["prefix_len"], 8)
        suf = np.array(wl.notes["suffix"])
        assert ((pre >= 1025) & (pre <= 1039)).all()
        assert ((suf >= 0) & (suf <= 512)).all()
        assert (c == pre + suf + 1).all()
    elif cfg == 5:
        assert B == 8 and c.min() >= 32768 and c.max() <= 131072
        assert (wl.num_heads, wl.num_kv_heads, wl.head_dim, wl.dtype) == (32, 8, 128, torch.bfloat16)


def test_deterministic_values():
    a, b = make_workload(1), make_workload(1)
    assert np.array_equal(a.free_order, b.free_order)
    ka, va = a.seq_kv(3)
    kb, vb = b.seq_kv(3)
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert torch.equal(a.q(), b.q())
    assert ka.shape == (100, 8, 64) and ka.dtype == torch.float16


def test_forked_samples_share_prefix_values():
    wl = make_workload(4)
    k0, _ = wl.seq_kv(0)
    k1, _ = wl.seq_kv(1)
    p = wl.notes["prefix_len"][0]
    assert torch.equal(k0[:p], k1[:p])
    assert not torch.equal(k0[p:p + 1], k1[p:p + 1]) or wl.ctx_lens[0] == p + 1


def test_custom_workload():
    wl = custom_workload([1, 16, 17], 16, 1, 64, dtype="bf16", seed=3)
    assert wl.ctx_lens.tolist() == [1, 16, 17] and wl.group == 16
    assert wl.num_blocks >= 1 + 1 + 2
