"""Synthetic prompts and prefix-dependent K/V for prefix-caching workloads.

Token ids are drawn uniformly from a 32000-word vocabulary.  In a model the K
and V of a token depend on every token before it; the stand-in here draws the
K/V of position p from a random stream keyed by a rolling hash of ids[0..p],
so two prompts share K/V exactly where they share a whole prefix (a block
reused after a different prefix would hold different values).  Values are
N(0, 1) in float32, rounded to the cache dtype, like the decode workloads.

The shapes follow the pages' two scenarios ("vLLM 核心概念", 前缀缓存): a
2000-token system prompt shared by many users' short queries, and a
multi-turn conversation whose history comes back in every turn.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np
import torch

VOCAB = 32000
_KIND_PREFIX_KV = 11
_KIND_PREFIX_Q = 12
_KIND_PROMPT = 13
_MASK = (1 << 63) - 1


def prompt_ids(seed: int, index: int, n: int) -> List[int]:
    """n token ids of prompt part ``index``."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, _KIND_PROMPT, index]))
    return rng.integers(0, VOCAB, n).astype(np.int64).tolist()


def prefix_hashes(ids: Sequence[int]) -> List[int]:
    """Rolling hash of every prefix ids[0..p]."""
    h, out = 0, []
    for t in ids:
        h = (h * 1000003 + int(t) + 1) & _MASK
        out.append(h)
    return out


def token_kv(seed: int, ids: Sequence[int], start: int, n: int, num_kv_heads: int, head_dim: int,
             dtype: torch.dtype) -> Tuple[torch.Tensor, torch.Tensor]:
    """K and V [n, Hkv, D] of positions start .. start+n-1 of the prompt ``ids`` (CPU)."""
    hs = prefix_hashes(ids[:start + n])[start:]
    k = np.empty((n, num_kv_heads, head_dim), dtype=np.float32)
    v = np.empty_like(k)
    for i, h in enumerate(hs):
        rng = np.random.default_rng(np.random.SeedSequence([seed, _KIND_PREFIX_KV, h]))
        kv = rng.standard_normal((2, num_kv_heads, head_dim), dtype=np.float32)
        k[i], v[i] = kv[0], kv[1]
    return torch.from_numpy(k).to(dtype), torch.from_numpy(v).to(dtype)


def queries(seed: int, request: int, n: int, num_heads: int, head_dim: int,
            dtype: torch.dtype) -> torch.Tensor:
    """Queries [n, H, D] of a request's n newly computed tokens (CPU)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, _KIND_PREFIX_Q, request, n]))
    q = rng.standard_normal((n, num_heads, head_dim), dtype=np.float32)
    return torch.from_numpy(q).to(dtype)


def system_prompt_requests(seed: int, num_requests: int, system_len: int = 2000,
                           query_lens: Tuple[int, int] = (16, 128)) -> List[List[int]]:
    """Prompts of requests sharing one system prompt, each with a private query of
    U{lo..hi} tokens."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, _KIND_PROMPT, 1 << 20]))
    system = prompt_ids(seed, 0, system_len)
    lens = rng.integers(query_lens[0], query_lens[1] + 1, num_requests)
    return [system + prompt_ids(seed, 1 + i, int(m)) for i, m in enumerate(lens)]
