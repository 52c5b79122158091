"""Pins of the cache oracle: hand-worked examples, round trips, invariances, ordering."""

import json
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import cache as C
from oracle import layout as L
from tests.conftest import GOLDEN


def test_layout_offsets_golden():
    g = json.load(open(os.path.join(GOLDEN, "layout_offsets.json")))
    nb, hkv, d, bs = g["num_blocks"], g["num_kv_heads"], g["head_dim"], g["block_size"]
    ids = np.arange(nb * hkv * bs * d, dtype=np.uint16).reshape(nb, hkv, bs, d)
    kflat = L.k_from_logical(ids).reshape(-1)
    vflat = L.v_from_logical(ids).reshape(-1)
    assert L.k_from_logical(ids).shape == L.k_physical_shape(nb, hkv, d, bs)
    assert L.v_from_logical(ids).shape == L.v_physical_shape(nb, hkv, d, bs)
    for e in g["k"]:
        assert kflat[e["offset"]] == ids[e["b"], e["h"], e["t"], e["d"]], e
    for e in g["v"]:
        assert vflat[e["offset"]] == ids[e["b"], e["h"], e["t"], e["d"]], e


@pytest.mark.parametrize("d", [64, 128])
def test_layout_round_trip(d):
    rng = np.random.default_rng(d)
    x = rng.integers(0, 65535, size=(3, 2, 16, d), dtype=np.uint16)
    assert np.array_equal(L.k_to_logical(L.k_from_logical(x)), x)
    assert np.array_equal(L.v_to_logical(L.v_from_logical(x)), x)


def test_cache_write_hand_example():
    kp, vp = C.empty_pool(3, 1, 2, block_size=4)
    k = np.array([[[1, 2]], [[3, 4]], [[5, 6]]], dtype=np.uint16)
    v = k + 100
    kp2, vp2 = C.cache_write(kp, vp, k, v, [5, -1, 8])
    # slot 5 = block 1 position 1; slot -1 skipped; slot 8 = block 2 position 0
    exp_k = np.zeros((3, 1, 4, 2), dtype=np.uint16)
    exp_k[1, 0, 1] = [1, 2]
    exp_k[2, 0, 0] = [5, 6]
    assert np.array_equal(kp2, exp_k)
    exp_v = np.zeros((3, 1, 4, 2), dtype=np.uint16)
    exp_v[1, 0, 1] = [101, 102]
    exp_v[2, 0, 0] = [105, 106]
    assert np.array_equal(vp2, exp_v)
    assert not kp.any()   # inputs untouched


def test_copy_blocks_hand_example():
    kp = np.arange(4 * 1 * 2 * 1, dtype=np.uint16).reshape(4, 1, 2, 1)
    vp = kp + 50
    k2, v2 = C.copy_blocks(kp, vp, [[0, 3], [2, 1]])
    assert k2[:, 0, :, 0].tolist() == [[0, 1], [4, 5], [4, 5], [0, 1]]
    assert v2[:, 0, :, 0].tolist() == [[50, 51], [54, 55], [54, 55], [50, 51]]


def test_page_unpage_round_trip_and_permutation_invariance():
    rng = np.random.default_rng(11)
    ctx, hkv, d, nb = 100, 2, 8, 20
    k = rng.standard_normal((ctx, hkv, d)).astype(np.float16).view(np.uint16)
    v = rng.standard_normal((ctx, hkv, d)).astype(np.float16).view(np.uint16)
    q = rng.standard_normal((4, d))
    ref = A.decode_attention(q, k.view(np.float16), v.view(np.float16), 0.3)
    for trial in range(3):
        table = rng.permutation(nb)[:7]
        kp, vp = C.empty_pool(nb, hkv, d, fill=0x7E00)      # NaN-poisoned pool
        kp, vp = C.scatter_sequence(kp, vp, table, k, v)
        gk, gv = C.gather_sequence(kp, vp, table, ctx)
        assert np.array_equal(gk, k) and np.array_equal(gv, v)
        out = A.decode_attention(q, gk.view(np.float16), gv.view(np.float16), 0.3)
        assert np.array_equal(out, ref)


def test_aliased_prefix_equals_duplicated_blocks():
    rng = np.random.default_rng(12)
    hkv, d, nb = 1, 8, 16
    prefix = rng.integers(0, 1000, size=(32, hkv, d), dtype=np.uint16)
    tails = [rng.integers(0, 1000, size=(5, hkv, d), dtype=np.uint16) for _ in range(2)]
    # aliased: both sequences point at blocks 3 and 7 for the prefix
    kp, vp = C.empty_pool(nb, hkv, d)
    kp, vp = C.scatter_sequence(kp, vp, [3, 7], prefix, prefix)
    kp, vp = C.cache_write(kp, vp, tails[0], tails[0], [9 * 16 + i for i in range(5)])
    kp, vp = C.cache_write(kp, vp, tails[1], tails[1], [11 * 16 + i for i in range(5)])
    # duplicated: each sequence owns a private copy of the prefix
    kd, vd = C.empty_pool(nb, hkv, d)
    kd, vd = C.scatter_sequence(kd, vd, [1, 2, 4], np.concatenate([prefix, tails[0]]),
                                np.concatenate([prefix, tails[0]]))
    kd, vd = C.scatter_sequence(kd, vd, [5, 6, 8], np.concatenate([prefix, tails[1]]),
                                np.concatenate([prefix, tails[1]]))
    for alias_t, dup_t in (([3, 7, 9], [1, 2, 4]), ([3, 7, 11], [5, 6, 8])):
        ga = C.gather_sequence(kp, vp, alias_t, 37)
        gd = C.gather_sequence(kd, vd, dup_t, 37)
        assert np.array_equal(ga[0], gd[0]) and np.array_equal(ga[1], gd[1])


def test_copy_before_write_is_required():
    """A planted ordering mistake: writing a sample's token into a still-shared
    block before its copy-on-write copy corrupts the sibling's view."""
    hkv, d, nb = 1, 4, 4
    kp, vp = C.empty_pool(nb, hkv, d)
    prefix = np.full((3, hkv, d), 7, dtype=np.uint16)
    kp, vp = C.scatter_sequence(kp, vp, [0], prefix, prefix)    # shared partial block 0
    tok_a = np.full((1, hkv, d), 1, dtype=np.uint16)
    tok_b = np.full((1, hkv, d), 2, dtype=np.uint16)
    # correct order: copy block 0 -> 2 (sample A's private copy), then write
    k1, v1 = C.copy_blocks(kp, vp, [[0, 2]])
    k1, v1 = C.cache_write(k1, v1, tok_a, tok_a, [2 * 16 + 3])
    k1, v1 = C.cache_write(k1, v1, tok_b, tok_b, [0 * 16 + 3])
    a_ok = C.gather_sequence(k1, v1, [2], 4)[0]
    b_ok = C.gather_sequence(k1, v1, [0], 4)[0]
    assert (a_ok[3] == 1).all() and (b_ok[3] == 2).all()
    # wrong order: B writes in place first, then A's copy carries B's token
    k2, v2 = C.cache_write(kp, vp, tok_b, tok_b, [0 * 16 + 3])
    k2, v2 = C.copy_blocks(k2, v2, [[0, 2]])
    a_bad = C.gather_sequence(k2, v2, [2], 4)[0]
    assert (a_bad[3] == 2).all()          # A now sees B's token: corrupted
    assert not np.array_equal(a_bad, a_ok)
