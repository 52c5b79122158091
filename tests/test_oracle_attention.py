"""Pins of the attention oracle: brute force, closed forms, invariants, mutations.

The brute force below is an independent pure-Python evaluation of
softmax(scale * q.K^T).V: Python floats, math.exp, no max shift, explicit
loops, and its own query-to-KV-head map written from the reading "query head
h reads KV head h // (H / Hkv)".
"""

import math

import numpy as np
import pytest

from oracle import attention as A


def brute_force(q, k, v, scale):
    H, D = len(q), len(q[0])
    ctx, Hkv = len(k), len(k[0])
    per_kv = H // Hkv
    out = []
    for h in range(H):
        g = h // per_kv
        w = []
        for t in range(ctx):
            dot = 0.0
            for d in range(D):
                dot += q[h][d] * k[t][g][d]
            w.append(math.exp(scale * dot))
        z = sum(w)
        row = []
        for d in range(D):
            acc = 0.0
            for t in range(ctx):
                acc += w[t] * v[t][g][d]
            row.append(acc / z)
        out.append(row)
    return np.array(out)


def _rand(rng, ctx, H, Hkv, D):
    q = rng.standard_normal((H, D))
    k = rng.standard_normal((ctx, Hkv, D))
    v = rng.standard_normal((ctx, Hkv, D))
    return q, k, v


@pytest.mark.parametrize("ctx,H,Hkv,D", [(1, 2, 2, 4), (7, 2, 2, 8), (17, 4, 2, 16), (40, 4, 1, 16),
                                         (33, 8, 2, 8), (16, 2, 1, 16)])
def test_brute_force(ctx, H, Hkv, D):
    rng = np.random.default_rng(1000 + ctx * 7 + H)
    q, k, v = _rand(rng, ctx, H, Hkv, D)
    scale = 1.0 / math.sqrt(D)
    ref = brute_force(q.tolist(), k.tolist(), v.tolist(), scale)
    got = A.decode_attention(q, k, v, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_brute_force_batch_with_torch_halves():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    ctxs = [3, 21]
    H, Hkv, D = 4, 2, 8
    q = torch.from_numpy(rng.standard_normal((2, H, D)).astype(np.float32)).to(torch.bfloat16)
    kv = {b: (torch.from_numpy(rng.standard_normal((c, Hkv, D)).astype(np.float32)).half(),
              torch.from_numpy(rng.standard_normal((c, Hkv, D)).astype(np.float32)).half())
          for b, c in enumerate(ctxs)}
    out = A.decode_batch(q, lambda b: kv[b], ctxs, 0.3)
    for b in range(2):
        ref = brute_force(q[b].double().tolist(), kv[b][0].double().tolist(),
                          kv[b][1].double().tolist(), 0.3)
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def test_single_token_is_exact_copy_of_v():
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 1, 4, 2, 16)
    out = A.decode_attention(q, k, v, 0.25)
    for h in range(4):
        assert np.array_equal(out[h], v[0, h // 2])


def test_zero_query_gives_mean_of_v():
    rng = np.random.default_rng(3)
    _, k, v = _rand(rng, 37, 4, 4, 8)
    out = A.decode_attention(np.zeros((4, 8)), k, v, 0.5)
    for h in range(4):
        np.testing.assert_allclose(out[h], np.mean(v[:, h, :], axis=0), rtol=1e-13, atol=1e-14)


def test_equal_keys_give_mean_of_v():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 29, 2, 1, 8)
    k[:] = k[0]
    out = A.decode_attention(q, k, v, 0.7)
    np.testing.assert_allclose(out[0], np.mean(v[:, 0, :], axis=0), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out[1], np.mean(v[:, 0, :], axis=0), rtol=1e-13, atol=1e-14)


def test_constant_v_is_reproduced():
    rng = np.random.default_rng(6)
    q, k, _ = _rand(rng, 50, 2, 2, 8)
    v = np.full((50, 2, 8), 1.75)
    out = A.decode_attention(q, k, v, 0.35)
    np.testing.assert_allclose(out, 1.75, rtol=1e-14)


def test_dominant_score_selects_its_value():
    rng = np.random.default_rng(7)
    D = 16
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    k = np.zeros((20, 1, D))
    k[11, 0, 0] = 30.0          # score +30 above every other token
    v = rng.standard_normal((20, 1, D))
    out = A.decode_attention(q, k, v, 1.0)
    bound = 19 * math.exp(-30) * np.abs(v).max() * 2
    assert np.max(np.abs(out[0] - v[11, 0])) < bound


@pytest.mark.parametrize("ctx", [1, 16, 513, 4096, 131072])
def test_weights_sum_to_one(ctx):
    rng = np.random.default_rng(ctx)
    q = rng.standard_normal(128)
    k = rng.standard_normal((ctx, 128))
    w = A.attention_weights(q, k, 1.0 / math.sqrt(128))
    assert abs(w.sum() - 1.0) < 1e-12
    assert np.all(w >= 0)


@pytest.mark.parametrize("seed", range(6))
def test_split_and_lse_merge_equals_unsplit(seed):
    rng = np.random.default_rng(100 + seed)
    ctx = int(rng.integers(2, 3000))
    D = 32
    q = rng.standard_normal(D) * 2
    k = rng.standard_normal((ctx, D))
    v = rng.standard_normal((ctx, D))
    cuts = sorted(set(rng.integers(1, ctx, size=int(rng.integers(1, 9))).tolist()))
    bounds = [0] + cuts + [ctx]
    states = [A.partial_state(q, k[a:b], v[a:b], 0.2) for a, b in zip(bounds[:-1], bounds[1:])]
    ms, ls, accs = zip(*states)
    whole = A.decode_attention(q[None, :], k[:, None, :], v[:, None, :], 0.2)[0]
    np.testing.assert_allclose(A.lse_merge(ms, ls, accs), whole, rtol=1e-12, atol=1e-13)
    # the same merge with maxima kept in log2 units
    ms2 = np.asarray(ms) / math.log(2.0)
    np.testing.assert_allclose(A.lse_merge(ms2, ls, accs, base=2.0), whole, rtol=1e-12, atol=1e-13)


def test_single_partition_merge_is_normalisation():
    rng = np.random.default_rng(9)
    acc = rng.standard_normal(8)
    np.testing.assert_allclose(A.lse_merge([3.0], [2.5], [acc]), acc / 2.5, rtol=1e-15)


# -- the pins above catch plausible mistakes planted in the oracle (on the CPU) -------
def _pins_pass():
    try:
        test_brute_force(17, 4, 2, 16)
        test_brute_force(40, 4, 1, 16)
        test_single_token_is_exact_copy_of_v()
        test_zero_query_gives_mean_of_v()
        test_constant_v_is_reproduced()
        test_dominant_score_selects_its_value()
        return True
    except AssertionError:
        return False


def _mutant_head_map(q, k, v, scale):
    qd = A._f64(q)
    H, D = qd.shape
    Hkv = k.shape[1]
    out = np.empty((H, D))
    for h in range(H):
        g = h % Hkv                       # wrong: interleaved instead of grouped
        out[h] = A.attention_weights(qd[h], A._f64(k[:, g, :]), scale) @ A._f64(v[:, g, :])
    return out


def _mutant_no_scale(q_h, k_g, scale):
    return A._f64(k_g) @ A._f64(q_h)      # dropped scale


def _mutant_drop_current(q_h, k_g, scale):
    s = scale * (A._f64(k_g) @ A._f64(q_h))
    s[-1] = -np.inf                       # forgets the current token
    return s


def _mutant_kv_swapped(q, k, v, scale):
    return _orig_decode(q, v, k, scale)   # transposed operands


_orig_decode = A.decode_attention


@pytest.mark.parametrize("name", ["head_map", "no_scale", "drop_current", "kv_swapped"])
def test_pins_catch_planted_mistakes(monkeypatch, name):
    assert _pins_pass()
    if name == "head_map":
        monkeypatch.setattr(A, "decode_attention", _mutant_head_map)
    elif name == "no_scale":
        monkeypatch.setattr(A, "scores", _mutant_no_scale)
    elif name == "drop_current":
        monkeypatch.setattr(A, "scores", _mutant_drop_current)
    elif name == "kv_swapped":
        monkeypatch.setattr(A, "decode_attention", _mutant_kv_swapped)
    assert not _pins_pass()


# -- several new tokens per sequence (prefill chunk / speculative verify) --------------
def brute_force_chunk(q, k, v, scale):
    """Independent loops: the last n of ctx tokens query, token i sees positions <= ctx-n+i."""
    n, H, D = len(q), len(q[0]), len(q[0][0])
    ctx, Hkv = len(k), len(k[0])
    per_kv = H // Hkv
    out = []
    for i in range(n):
        pos = ctx - n + i
        rows = []
        for h in range(H):
            g = h // per_kv
            w = []
            for t in range(pos + 1):
                dot = 0.0
                for d in range(D):
                    dot += q[i][h][d] * k[t][g][d]
                w.append(math.exp(scale * dot))
            z = sum(w)
            rows.append([sum(w[t] * v[t][g][d] for t in range(pos + 1)) / z for d in range(D)])
        out.append(rows)
    return np.array(out)


@pytest.mark.parametrize("n,ctx,H,Hkv,D", [(1, 1, 2, 2, 4), (3, 3, 2, 1, 8), (4, 9, 4, 2, 8),
                                           (6, 20, 8, 2, 4), (5, 17, 2, 2, 16)])
def test_chunk_brute_force(n, ctx, H, Hkv, D):
    rng = np.random.default_rng(4000 + 31 * n + ctx)
    q = rng.standard_normal((n, H, D))
    k = rng.standard_normal((ctx, Hkv, D))
    v = rng.standard_normal((ctx, Hkv, D))
    scale = 1.0 / math.sqrt(D)
    ref = brute_force_chunk(q.tolist(), k.tolist(), v.tolist(), scale)
    np.testing.assert_allclose(A.chunk_attention(q, k, v, scale), ref, rtol=1e-12, atol=1e-13)


def test_chunk_of_one_token_is_decode():
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 23, 8, 2, 16)
    np.testing.assert_array_equal(A.chunk_attention(q[None], k, v, 0.2)[0],
                                  A.decode_attention(q, k, v, 0.2))


def test_whole_prompt_equals_torch_causal_attention():
    """n = ctx: the chunk is the whole prompt, i.e. plain causal self-attention
    (torch's scaled_dot_product_attention, float64, is_causal)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    ctx, H, Hkv, D = 37, 8, 2, 16
    q = rng.standard_normal((ctx, H, D))
    k = rng.standard_normal((ctx, Hkv, D))
    v = rng.standard_normal((ctx, Hkv, D))
    scale = 0.125
    tq = torch.from_numpy(q).permute(1, 0, 2)                       # [H, ctx, D]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(H // Hkv, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(H // Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                           scale=scale)
    np.testing.assert_allclose(A.chunk_attention(q, k, v, scale), ref.permute(1, 0, 2).numpy(),
                               rtol=1e-11, atol=1e-12)


def test_chunking_a_prompt_does_not_change_its_outputs():
    rng = np.random.default_rng(13)
    ctx, H, Hkv, D = 41, 4, 2, 8
    q = rng.standard_normal((ctx, H, D))
    k = rng.standard_normal((ctx, Hkv, D))
    v = rng.standard_normal((ctx, Hkv, D))
    whole = A.chunk_attention(q, k, v, 0.3)
    parts, start = [], 0
    for size in (16, 1, 9, 15):
        end = start + size
        parts.append(A.chunk_attention(q[start:end], k[:end], v[:end], 0.3))
        start = end
    np.testing.assert_allclose(np.concatenate(parts), whole, rtol=1e-13, atol=1e-14)


def test_chunk_queries_see_nothing_after_their_position():
    rng = np.random.default_rng(14)
    n, ctx, H, Hkv, D = 5, 12, 4, 2, 8
    q = rng.standard_normal((n, H, D))
    k = rng.standard_normal((ctx, Hkv, D))
    v = rng.standard_normal((ctx, Hkv, D))
    base = A.chunk_attention(q, k, v, 0.4)
    for i in range(n):
        pos = ctx - n + i
        k2, v2 = k.copy(), v.copy()
        k2[pos + 1:] += 3.0
        v2[pos + 1:] -= 5.0
        assert np.array_equal(A.chunk_attention(q, k2, v2, 0.4)[i], base[i])
        k3 = k.copy()
        k3[pos] += 3.0
        assert not np.allclose(A.chunk_attention(q, k3, v, 0.4)[i], base[i])


def test_chunk_batch_rows_follow_q_starts():
    rng = np.random.default_rng(15)
    H, Hkv, D = 4, 2, 8
    ctx = [9, 3, 20]
    n = [2, 0, 5]
    starts = np.concatenate([[0], np.cumsum(n)])
    kv = [(rng.standard_normal((c, Hkv, D)), rng.standard_normal((c, Hkv, D))) for c in ctx]
    q = rng.standard_normal((int(starts[-1]), H, D))
    out = A.chunk_batch(q, starts, lambda b: kv[b], ctx, 0.3)
    for b in range(3):
        lo, hi = starts[b], starts[b + 1]
        if hi > lo:
            np.testing.assert_array_equal(out[lo:hi], A.chunk_attention(q[lo:hi], *kv[b], 0.3))


def _chunk_pins_pass():
    try:
        test_chunk_brute_force(4, 9, 4, 2, 8)
        test_chunk_brute_force(6, 20, 8, 2, 4)
        test_chunk_queries_see_nothing_after_their_position()
        return True
    except AssertionError:
        return False


def _make_chunk_mutant(shift=0, causal=True):
    def mutant(q, k, v, scale):
        qd = A._f64(q)
        n, H, D = qd.shape
        ctx, Hkv = k.shape[0], k.shape[1]
        G = H // Hkv
        out = np.empty((n, H, D))
        for i in range(n):
            visible = min(ctx, max(1, ctx - n + i + 1 + shift)) if causal else ctx
            for h in range(H):
                g = h // G
                kg, vg = A._f64(k[:visible, g, :]), A._f64(v[:visible, g, :])
                out[i, h] = A.attention_weights(qd[i, h], kg, scale) @ vg
        return out
    return mutant


@pytest.mark.parametrize("name", ["excludes_self", "sees_next", "not_causal"])
def test_chunk_pins_catch_planted_mistakes(monkeypatch, name):
    assert _chunk_pins_pass()
    mutant = {"excludes_self": _make_chunk_mutant(shift=-1),
              "sees_next": _make_chunk_mutant(shift=1),
              "not_causal": _make_chunk_mutant(causal=False)}[name]
    monkeypatch.setattr(A, "chunk_attention", mutant)
    assert not _chunk_pins_pass()
