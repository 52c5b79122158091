"""Decode attention by its plain definition, in float64.  TEST INFRASTRUCTURE ONLY.

What is computed, and where the pages fix it:

* At a decode step the model computes the query, key and value of the current
  token only and reuses the cached keys and values of every earlier token
  ("vLLM 核心概念", section "为什么需要 KV Cache？"); each decode step therefore
  reads the whole history ("PagedAttention 实战", section "Decode：逐 token 生成输出";
  "理解 vLLM PagedAttention", section 七).  So the single query of sequence b
  attends over all ctx_b cached positions, the current token included, and
  nothing past ctx_b.
* The pages never write the softmax out.  The plain reading, which nothing on
  them contradicts, is scaled dot-product attention with the caller's scale:
      s_t = scale * <q_h, K[t, g]>,  out_h = sum_t softmax(s)_t * V[t, g].
* Query heads and KV heads: the pages only name a "KV-head group"
  ("PagedAttention 实战", section "2026 年的新变化").  Reading: with
  G = H / Hkv, query head h reads KV head floor(h / G).
* Long contexts split into partitions whose partial softmax states are merged
  by log-sum-exp (the "sequence split" of the same section): ``partial_state``
  and ``lse_merge`` below state that merge in its textbook form.
* Several new tokens per sequence (a prefill chunk, a speculative verify):
  ``chunk_attention`` / ``chunk_batch``, the causal reading stated with them.

Everything is upcast exactly to float64 before any arithmetic.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """float64 copy of a numpy array or a CPU torch tensor (any float dtype)."""
    if hasattr(x, "detach"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def scores(q_h, k_g, scale: float) -> np.ndarray:
    """s_t = scale * <q_h, k_t> for every cached token t; q_h [D], k_g [ctx, D]."""
    return scale * (_f64(k_g) @ _f64(q_h))


def attention_weights(q_h, k_g, scale: float) -> np.ndarray:
    """softmax over the context of the scaled scores (max-shifted for range)."""
    s = scores(q_h, k_g, scale)
    p = np.exp(s - s.max())
    return p / p.sum()


def decode_attention(q, k, v, scale: float) -> np.ndarray:
    """One sequence: q [H, D], k and v [ctx, Hkv, D]  ->  out [H, D] (float64)."""
    qd = _f64(q)
    H, D = qd.shape
    Hkv = k.shape[1]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = H // Hkv
    out = np.empty((H, D), dtype=np.float64)
    for g in range(Hkv):
        kg = _f64(k[:, g, :])
        vg = _f64(v[:, g, :])
        for h in range(g * G, (g + 1) * G):
            out[h] = attention_weights(qd[h], kg, scale) @ vg
    return out


def decode_batch(q, seq_kv, ctx_lens, scale: float, seqs=None) -> np.ndarray:
    """out [B, H, D] for the sequences ``seqs`` (default all); ``seq_kv(b)`` -> (k, v)."""
    qd = _f64(q)
    B, H, D = qd.shape
    seqs = range(B) if seqs is None else seqs
    out = np.full((B, H, D), np.nan)
    for b in seqs:
        k, v = seq_kv(b)
        if k.shape[0] != int(ctx_lens[b]):
            raise ValueError(f"sequence {b}: {k.shape[0]} cached tokens, context {ctx_lens[b]}")
        out[b] = decode_attention(qd[b], k, v, scale)
    return out


def partial_state(q_h, k_g, v_g, scale: float):
    """Unnormalised softmax state of one query over a token range (natural log domain).

    Returns (m, l, acc): m = max_t s_t, l = sum_t exp(s_t - m),
    acc = sum_t exp(s_t - m) * v_t.  The normalised output of the range is acc / l.
    """
    s = scores(q_h, k_g, scale)
    m = s.max()
    p = np.exp(s - m)
    return m, p.sum(), p @ _f64(v_g)


def lse_merge(ms, ls, accs, base: float = np.e) -> np.ndarray:
    """Merge partial states (m_p, l_p, acc_p) into the normalised output.

    With M = max_p m_p and w_p = base**(m_p - M):
        out = sum_p w_p acc_p / sum_p w_p l_p.
    ``base`` is the base the states' maxima are expressed in (e for
    ``partial_state``; 2 for states kept in log2 units).
    """
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    accs = np.asarray(accs, dtype=np.float64)
    M = ms.max()
    w = np.power(base, ms - M)
    return (w @ accs) / (w @ ls)


# ---- several new tokens per sequence: a prefill chunk, or a speculative verify ----------
#
# A long prompt is prefilled in chunks: each chunk's tokens get their keys and
# values cached and attend to everything before them, so later chunks build on
# the cache the earlier ones left ("vLLM 核心概念", section "Chunked Prefill";
# "PagedAttention 实战", section "Chunked Prefill：长 prompt 不要一次吃完全部预算").
# Verifying the draft tokens of speculative decoding runs the main model over
# several new tokens at once ("vLLM 核心概念", section "推测解码（Speculative
# Decoding）").  Both are the same computation: the last
# n of a sequence's ctx cached tokens are queries, and query i (position
# ctx - n + i) attends over positions 0 .. ctx - n + i -- the causal reading
# that the prompt's tokens see only what precedes them (and themselves).
# With n = 1 it is exactly ``decode_attention``.


def chunk_attention(q, k, v, scale: float) -> np.ndarray:
    """One sequence: q [n, H, D] (its last n tokens), k and v [ctx, Hkv, D], n <= ctx
    ->  out [n, H, D] (float64); query i attends over k[: ctx - n + i + 1]."""
    qd = _f64(q)
    n, H, D = qd.shape
    ctx, Hkv = k.shape[0], k.shape[1]
    if n > ctx:
        raise ValueError(f"{n} new tokens but only {ctx} cached")
    if H % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = H // Hkv
    out = np.empty((n, H, D), dtype=np.float64)
    for g in range(Hkv):
        kg = _f64(k[:, g, :])
        vg = _f64(v[:, g, :])
        for i in range(n):
            visible = ctx - n + i + 1
            for h in range(g * G, (g + 1) * G):
                out[i, h] = attention_weights(qd[i, h], kg[:visible], scale) @ vg[:visible]
    return out


def chunk_batch(q, q_starts, seq_kv, ctx_lens, scale: float, seqs=None) -> np.ndarray:
    """Packed queries q [total, H, D]; sequence b owns rows q_starts[b] .. q_starts[b+1]
    and ``seq_kv(b)`` -> (k, v) of its ctx_lens[b] cached tokens.  Returns out
    [total, H, D] (NaN in the rows of sequences not in ``seqs``)."""
    qd = _f64(q)
    out = np.full(qd.shape, np.nan)
    B = len(ctx_lens)
    seqs = range(B) if seqs is None else seqs
    for b in seqs:
        lo, hi = int(q_starts[b]), int(q_starts[b + 1])
        if hi == lo:
            continue
        k, v = seq_kv(b)
        if k.shape[0] != int(ctx_lens[b]):
            raise ValueError(f"sequence {b}: {k.shape[0]} cached tokens, context {ctx_lens[b]}")
        out[lo:hi] = chunk_attention(qd[lo:hi], k, v, scale)
    return out
