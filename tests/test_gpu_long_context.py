"""GPU parity of long-context split decode: many context partitions per sequence,
merged by log-sum-exp ("PagedAttention 实战", section "2026 年的新变化": sequence
split).

* Single long sequences whose launches take 512- or 1024-token partitions, so one
  sequence has 79 to 256 partitions and the separate merge walks them in several
  64-partition rounds.  The step (``pa_decode_step``), ``pa_decode``, the two
  stage calls and ``pa_decode_partitioned`` give the same bits, within tolerance
  of the oracle.
* The long-context workload (8 sequences of 32k-128k tokens) with its stated
  split, 512-token partitions (``pa_decode_partitioned``), against the oracle on
  every sequence; the per-launch choice (4096-token partitions there) is the
  step's, checked in the workload parity tests.
"""

import numpy as np
import pytest
import torch

from tests.gpu_harness import build_device, check_close, oracle_out, run_step, say
from workloads import custom_workload, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import paged_kv_cache_385_amd._native as N
    N.lib()


LONG = [
    # ctx, H, Hkv, D, dtype, partition tokens the launch chooses, partitions of the longest
    ([40000], 8, 1, 128, "bf16", 512, 79),
    ([131072], 64, 8, 128, "bf16", 512, 256),
    ([100000, 131072], 32, 8, 128, "f16", 1024, 128),
]


@pytest.mark.parametrize("ctx,H,Hkv,D,dt,pt,parts", LONG)
def test_many_partitions_merge(ctx, H, Hkv, D, dt, pt, parts):
    from paged_kv_cache_385_amd import (alloc_workspace, decode, decode_attention, decode_merge,
                                        decode_partitioned)
    wl = custom_workload(ctx, H, Hkv, D, dtype=dt, seed=sum(ctx) % 1000 + H)
    assert -(-max(ctx) // pt) == parts and parts > 64
    say(f"long context {ctx}, H={H} Hkv={Hkv} D={D} {dt}: {pt}-token partitions, {parts} of them")
    cache, segs = build_device(wl)
    out_step, batch = run_step(wl, cache, segs)
    out_step = out_step.clone()
    ref = oracle_out(wl, segs)
    check_close(out_step, ref, wl.dtype, label=f"step, {parts} partitions")
    q = wl.q().cuda()
    mx = int(wl.ctx_lens.max())
    ws = alloc_workspace(wl.num_seqs, H, D, mx)
    one = decode(cache.k_cache, cache.v_cache, q, batch.tables_d, batch.ctx_d, mx, wl.scale,
                 workspace=ws).clone()
    two = decode_attention(cache.k_cache, cache.v_cache, q, batch.tables_d, batch.ctx_d, mx,
                           wl.scale, workspace=ws)
    two = decode_merge(cache.k_cache, cache.v_cache, batch.ctx_d, mx, two, workspace=ws).clone()
    fixed = decode_partitioned(cache.k_cache, cache.v_cache, q, batch.tables_d, batch.ctx_d, mx,
                               wl.scale, pt, workspace=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(one, out_step)
    assert torch.equal(two, out_step)
    assert torch.equal(fixed, out_step)
    # another partition length: another rounding of the merge, the same result within tolerance
    other = 4096 if pt != 4096 else 512
    alt = decode_partitioned(cache.k_cache, cache.v_cache, q, batch.tables_d, batch.ctx_d, mx,
                             wl.scale, other, workspace=ws)
    torch.cuda.synchronize()
    check_close(alt, ref, wl.dtype, label=f"{other}-token partitions")
    # every call leaves the counter region zero: the merge counters and the counter that
    # hands out the item list's places after the first round of workgroups
    from paged_kv_cache_385_amd.ops import workspace_counter_bytes
    c = workspace_counter_bytes(wl.num_seqs, H)
    assert int(ws[:c].count_nonzero()) == 0
    assert int(batch.workspace[:c].count_nonzero()) == 0


def test_long_context_workload_with_512_token_partitions():
    from paged_kv_cache_385_amd import alloc_workspace, decode, decode_partitioned
    from paged_kv_cache_385_amd.ops import workspace_counter_bytes
    wl = make_workload(5)
    parts = -(-wl.ctx_lens // 512)
    say(f"workload 5 with 512-token partitions: {parts.min()}..{parts.max()} per sequence")
    cache, segs = build_device(wl)
    out_step, batch = run_step(wl, cache, segs)
    out_step = out_step.clone()
    q = wl.q().cuda()
    mx = int(wl.ctx_lens.max())
    ws = alloc_workspace(wl.num_seqs, wl.num_heads, wl.head_dim, mx)
    c = workspace_counter_bytes(wl.num_seqs, wl.num_heads)
    ws[c:].view(torch.float32).fill_(float("nan"))            # states the pass must overwrite
    out = torch.full_like(q, float("nan"))
    decode_partitioned(cache.k_cache, cache.v_cache, q, batch.tables_d, batch.ctx_d, mx, wl.scale,
                       512, out=out, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle_out(wl, segs)
    check_close(out, ref, wl.dtype, label="workload 5, 512-token partitions")
    # the per-launch choice through pa_decode_partitioned(0) is pa_decode, and the step's
    auto = decode_partitioned(cache.k_cache, cache.v_cache, q, batch.tables_d, batch.ctx_d, mx,
                              wl.scale, 0, workspace=ws).clone()
    plain = decode(cache.k_cache, cache.v_cache, q, batch.tables_d, batch.ctx_d, mx, wl.scale,
                   workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(auto, plain) and torch.equal(auto, out_step)
    assert int(ws[:c].count_nonzero()) == 0
    assert int(batch.workspace[:c].count_nonzero()) == 0
