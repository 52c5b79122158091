"""The five synthetic decode workloads, drawn from fixed seeds.

Every workload is one decode step of one attention layer:

* a *setup* trace of block-manager operations (add a sequence, append tokens
  to it, fork it) that builds the cache state before the step, and
* the *step* itself: one new token appended to every sequence, in sequence
  order, followed by attention of each sequence's query over its whole
  context (the cached history plus the new token).

Token values come in *segments*.  A segment is a run of tokens whose K and V
vectors are drawn from one keyed random stream; a sequence's logical K/V is
the concatenation of the segment slices appended to it, in order.  Forked
sequences inherit their parent's slices, so aliased prefixes really hold the
same values.  Streams are keyed by ``(seed, kind, index)`` so any one segment
can be regenerated alone.

Values are drawn N(0, 1) in float32 and rounded to the workload dtype with
round-to-nearest-even (torch's CPU conversion); the rounded values are what
every consumer sees.

Workload shapes (the five decode workloads the pages' explainers motivate:
a tiny case, a 7B-like MHA layer, a 70B-like GQA-8 layer, shared-prefix
parallel sampling and long-context split decode) are listed in ``_SPECS``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

import numpy as np
import torch

BLOCK_SIZE = 16
CONFIG_IDS = (1, 2, 3, 4, 5)

# stream kinds for SeedSequence keys
_KIND_SEGMENT = 1
_KIND_Q = 2
_KIND_STEP_TOKEN = 3
_KIND_STEP_Q = 4
_KIND_CHUNK_Q = 5

_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


def _seed_for(cfg_id: int) -> int:
    return 385 * 10 + cfg_id


@dataclass
class Workload:
    cfg_id: int
    name: str
    dtype_name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    seed: int
    num_blocks: int
    free_order: np.ndarray          # int32 [num_blocks], pop order of the free list
    ctx_lens: np.ndarray            # int64 [num_seqs], context incl. the step's new token
    setup: List[tuple]              # ("add", s) | ("append", s, seg, start, n) | ("fork", p, c)
    step: List[tuple]               # ("append", s, seg, start, 1) for every sequence, in order
    seg_lengths: Dict[int, int]
    seq_slices: Dict[int, List[Tuple[int, int, int]]]  # seq -> [(seg, start, n)] logical order
    block_size: int = BLOCK_SIZE
    notes: Dict[str, object] = field(default_factory=dict)

    @property
    def dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype_name]

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def max_context_len(self) -> int:
        return int(self.ctx_lens.max())

    def segment_kv(self, seg_id: int) -> Tuple[torch.Tensor, torch.Tensor]:
        """K and V of one segment, each [len, Hkv, D] in the workload dtype (CPU)."""
        n = self.seg_lengths[seg_id]
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, _KIND_SEGMENT, seg_id]))
        shape = (n, self.num_kv_heads, self.head_dim)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        return (torch.from_numpy(k).to(self.dtype), torch.from_numpy(v).to(self.dtype))

    def seq_kv(self, seq: int, cache: Dict[int, Tuple[torch.Tensor, torch.Tensor]] | None = None
               ) -> Tuple[torch.Tensor, torch.Tensor]:
        """Logical (never paged) K and V of a sequence, [ctx, Hkv, D]."""
        ks, vs = [], []
        for seg, start, n in self.seq_slices[seq]:
            if cache is not None and seg in cache:
                k, v = cache[seg]
            else:
                k, v = self.segment_kv(seg)
                if cache is not None:
                    cache[seg] = (k, v)
            ks.append(k[start:start + n])
            vs.append(v[start:start + n])
        return torch.cat(ks, 0), torch.cat(vs, 0)

    def q(self) -> torch.Tensor:
        """Query of the step, [B, H, D] in the workload dtype (CPU)."""
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, _KIND_Q]))
        q = rng.standard_normal((self.num_seqs, self.num_heads, self.head_dim), dtype=np.float32)
        return torch.from_numpy(q).to(self.dtype)

    def chunk_q(self, q_lens: Sequence[int]) -> torch.Tensor:
        """Queries of the last q_lens[b] tokens of every sequence, packed in sequence
        order: [sum(q_lens), H, D] in the workload dtype (CPU)."""
        lens = [int(n) for n in q_lens]
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, _KIND_CHUNK_Q, *lens]))
        q = rng.standard_normal((sum(lens), self.num_heads, self.head_dim), dtype=np.float32)
        return torch.from_numpy(q).to(self.dtype)

    def kv_bytes(self) -> int:
        """Bytes of K and V one decode step must read: every context token, both caches."""
        elem = 2
        return int(self.ctx_lens.sum()) * 2 * self.num_kv_heads * self.head_dim * elem


def new_token_kv(seed: int, step: int, num_seqs: int, num_kv_heads: int, head_dim: int,
                 dtype: torch.dtype) -> Tuple[torch.Tensor, torch.Tensor]:
    """k, v [B, Hkv, D] of the new tokens of an extra decode step ``step`` (bench growth)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, _KIND_STEP_TOKEN, step]))
    k = rng.standard_normal((num_seqs, num_kv_heads, head_dim), dtype=np.float32)
    v = rng.standard_normal((num_seqs, num_kv_heads, head_dim), dtype=np.float32)
    return torch.from_numpy(k).to(dtype), torch.from_numpy(v).to(dtype)


def _pool_size(block_counts: Sequence[int], slack: float = 1.1) -> int:
    return int(math.ceil(slack * sum(block_counts)))


def _blocks_for(tokens: int) -> int:
    # workload sizing only (how big the pool must be), not the allocator
    return -(-tokens // BLOCK_SIZE)


def _independent(cfg_id: int, name: str, dtype: str, ctx: np.ndarray, H: int, Hkv: int, D: int,
                 seed: int, rng: np.random.Generator, num_blocks: int | None = None,
                 grow: int = 0) -> Workload:
    """Sequences that share nothing: seq b owns segment b holding all ctx_b tokens."""
    ctx = np.asarray(ctx, dtype=np.int64)
    B = len(ctx)
    if num_blocks is None:
        num_blocks = _pool_size([_blocks_for(int(c) + grow) for c in ctx])
    free_order = rng.permutation(num_blocks).astype(np.int32)
    setup, step = [], []
    seg_lengths, seq_slices = {}, {}
    for b in range(B):
        c = int(ctx[b])
        seg_lengths[b] = c
        seq_slices[b] = [(b, 0, c)]
        setup.append(("add", b))
        if c > 1:
            setup.append(("append", b, b, 0, c - 1))
        step.append(("append", b, b, c - 1, 1))
    return Workload(cfg_id=cfg_id, name=name, dtype_name=dtype, num_seqs=B, num_heads=H,
                    num_kv_heads=Hkv, head_dim=D, scale=1.0 / math.sqrt(D), seed=seed,
                    num_blocks=num_blocks, free_order=free_order, ctx_lens=ctx, setup=setup,
                    step=step, seg_lengths=seg_lengths, seq_slices=seq_slices)


def _shared_prefix(seed: int, rng: np.random.Generator, prompts: int = 16, samples: int = 8,
                   prefix: int = 1024, suffix_max: int = 512, extra_max: int = 15, H: int = 32,
                   D: int = 128, dtype: str = "f16", grow: int = 0,
                   Hkv: int | None = None) -> Workload:
    """Parallel sampling over a shared prompt prefix.

    Prompt p's prefix holds ``prefix + r_p`` tokens, r_p ~ U{1..extra_max}, so
    its last block is partially filled and shared by all ``samples`` children.
    Each sample then appends a private suffix of U{0..suffix_max} tokens and
    finally the step's new token.  ``extra_max = 0`` gives the literal
    block-aligned prefix (r_p = 0).  ``Hkv`` KV heads (default ``H``: one query
    head per KV head).
    """
    B = prompts * samples
    extras = (rng.integers(1, extra_max, size=prompts, endpoint=True) if extra_max > 0
              else np.zeros(prompts, dtype=np.int64))
    suffix = rng.integers(0, suffix_max, size=B, endpoint=True)
    prefix_len = prefix + extras
    ctx = np.array([prefix_len[b // samples] + suffix[b] + 1 for b in range(B)], dtype=np.int64)
    # unique demand: full shared prefix blocks once per prompt, the rest per sample
    demand = 0
    for p in range(prompts):
        demand += int(prefix_len[p]) // BLOCK_SIZE
    for b in range(B):
        demand += _blocks_for(int(ctx[b]) + grow) - int(prefix_len[b // samples]) // BLOCK_SIZE
    num_blocks = _pool_size([demand])
    free_order = rng.permutation(num_blocks).astype(np.int32)
    setup, step = [], []
    seg_lengths, seq_slices = {}, {}
    # segment ids: prompt prefixes 0..prompts-1, private tails prompts..prompts+B-1
    for p in range(prompts):
        seg_lengths[p] = int(prefix_len[p])
        parent = p * samples
        setup.append(("add", parent))
        setup.append(("append", parent, p, 0, int(prefix_len[p])))
        for s in range(1, samples):
            setup.append(("fork", parent, parent + s))
    for b in range(B):
        seg = prompts + b
        seg_lengths[seg] = int(suffix[b]) + 1
        p = b // samples
        seq_slices[b] = [(p, 0, int(prefix_len[p])), (seg, 0, int(suffix[b]) + 1)]
        if suffix[b] > 0:
            setup.append(("append", b, seg, 0, int(suffix[b])))
        step.append(("append", b, seg, int(suffix[b]), 1))
    wl = Workload(cfg_id=4, name="shared-prefix parallel sampling", dtype_name=dtype, num_seqs=B,
                  num_heads=H, num_kv_heads=H if Hkv is None else Hkv, head_dim=D,
                  scale=1.0 / math.sqrt(D), seed=seed,
                  num_blocks=num_blocks, free_order=free_order, ctx_lens=ctx, setup=setup,
                  step=step, seg_lengths=seg_lengths, seq_slices=seq_slices)
    wl.notes.update(prompts=prompts, samples=samples, prefix_len=prefix_len.tolist(),
                    suffix=suffix.tolist())
    return wl


def make_workload(cfg_id: int, grow: int = 0, **overrides) -> Workload:
    """Build workload ``cfg_id`` (1..5).  ``grow`` adds pool room for that many extra steps."""
    seed = overrides.pop("seed", _seed_for(cfg_id))
    rng = np.random.default_rng(seed)
    if cfg_id == 1:
        ctx = np.array([17, 33, 64, 100], dtype=np.int64)
        return _independent(1, "tiny paged decode", "f16", ctx, 8, 8, 64, seed, rng,
                            num_blocks=64 if grow == 0 else None, grow=grow)
    if cfg_id == 2:
        ctx = rng.integers(128, 2048, size=64, endpoint=True)
        return _independent(2, "7B-shaped MHA decode layer", "f16", ctx, 32, 32, 128, seed, rng,
                            grow=grow)
    if cfg_id == 3:
        z = rng.standard_normal(128)
        ctx = np.clip(np.rint(1024.0 * np.exp(z)), 16, 4096).astype(np.int64)
        wl = _independent(3, "70B-shaped GQA-8 decode layer", "bf16", ctx, 64, 8, 128, seed, rng,
                          grow=grow)
        wl.notes["lognormal_sigma"] = 1.0
        return wl
    if cfg_id == 4:
        return _shared_prefix(seed, rng, grow=grow, **overrides)
    if cfg_id == 5:
        ctx = rng.integers(32768, 131072, size=8, endpoint=True)
        return _independent(5, "long-context split decode", "bf16", ctx, 32, 8, 128, seed, rng,
                            grow=grow)
    raise ValueError(f"unknown workload {cfg_id}")


def custom_workload(ctx: Sequence[int], num_heads: int, num_kv_heads: int, head_dim: int,
                    dtype: str = "f16", seed: int = 0, num_blocks: int | None = None,
                    grow: int = 0) -> Workload:
    """Independent sequences with explicit lengths, for edge cases."""
    rng = np.random.default_rng(seed)
    return _independent(0, "custom", dtype, np.asarray(ctx, dtype=np.int64), num_heads,
                        num_kv_heads, head_dim, seed, rng, num_blocks=num_blocks, grow=grow)
