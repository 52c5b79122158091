"""GPU parity of decode with more than 16 query heads per KV head (MQA-like groups).

One matrix-core tile of the decode pass holds 16 query heads; wider groups run the
several-token kernels with one query per sequence.  Outputs within 2e-3 (float16) /
1e-2 (bfloat16) of the float64 oracle, through the decode step (cache write, then
attention), pa_decode, and the two-stage calls.
"""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import fp8 as OF
from tests.gpu_harness import SegCache, build_device, check_close, oracle_out, run_step, say
from workloads import custom_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import paged_kv_cache_385_amd._native as N
    N.lib()


WIDE = [
    # ctx list, H, Hkv, D, dtype
    ([1, 17, 600, 3000], 32, 1, 128, "bf16"),    # G=32: two column tiles, key partitions
    ([5, 250, 1100], 64, 2, 128, "f16"),          # G=32
    ([33, 700, 1500, 9], 64, 1, 128, "f16"),      # G=64: 48 + 16 columns
    ([40, 2000], 128, 1, 64, "bf16"),             # G=128: the wide kernel
]


@pytest.mark.parametrize("ctx,H,Hkv,D,dt", WIDE)
def test_wide_group_step(ctx, H, Hkv, D, dt):
    wl = custom_workload(ctx, H, Hkv, D, dtype=dt, seed=H + D + len(ctx))
    say(f"wide group G={H // Hkv}: ctx={ctx} H={H} Hkv={Hkv} D={D} {dt}")
    cache, segs = build_device(wl)
    out, _ = run_step(wl, cache, segs)
    check_close(out, oracle_out(wl, segs), wl.dtype, label=f"G={H // Hkv} step")


def test_wide_group_entry_points_agree():
    """After the step, pa_decode and pa_decode_attention + pa_decode_merge on the same
    cache give the step's output bit for bit (the same kernels, in the same order)."""
    from paged_kv_cache_385_amd import decode, decode_attention, decode_merge
    wl = custom_workload([1, 17, 600, 3000], 32, 1, 128, dtype="bf16", seed=7)
    cache, segs = build_device(wl)
    out, batch = run_step(wl, cache, segs)
    q = wl.q().cuda()
    mc = int(wl.ctx_lens.max())
    d = decode(cache.k_cache, cache.v_cache, q, batch.tables_d, batch.ctx_d, mc, wl.scale,
               workspace=batch.workspace)
    two = torch.full_like(out, float("nan"))
    decode_attention(cache.k_cache, cache.v_cache, q, batch.tables_d, batch.ctx_d, mc, wl.scale,
                     out=two, workspace=batch.workspace)
    decode_merge(cache.k_cache, cache.v_cache, batch.ctx_d, mc, two, workspace=batch.workspace)
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.int16), out.view(torch.int16))
    assert torch.equal(two.view(torch.int16), out.view(torch.int16))


def test_wide_group_fp8_step():
    from paged_kv_cache_385_amd import DecodeBatch, PagedKVCache
    wl = custom_workload([3, 300, 2500], 32, 1, 128, dtype="bf16", seed=12)
    ks = np.array([0.01], np.float32)
    vs = np.array([0.015], np.float32)
    segs = SegCache(wl)
    cache = PagedKVCache(wl.num_blocks, 1, 128, wl.dtype, "cuda", free_order=wl.free_order,
                         fill_bits=0x7F, kv_scales=(ks, vs))
    cache.apply_trace(wl.setup, segs.tokens)
    sids = [op[1] for op in wl.step]
    batch = DecodeBatch(cache, sids, 32, wl.scale, -(-int(wl.ctx_lens.max()) // 16))
    k_new, v_new = (torch.cat(t).cuda() for t in zip(*(segs.tokens(op[2], op[3], 1) for op in wl.step)))
    out = batch.step(k_new, v_new, wl.q().cuda())
    torch.cuda.synchronize()

    def seq_kv(b):
        k, v = wl.seq_kv(b, segs)
        kq = OF.dequantize(OF.quantize(k.float().numpy(), ks[None, :, None]), ks[None, :, None])
        vq = OF.dequantize(OF.quantize(v.float().numpy(), vs[None, :, None]), vs[None, :, None])
        return kq, vq
    ref = OA.decode_batch(wl.q(), seq_kv, wl.ctx_lens, wl.scale)
    check_close(out, ref, wl.dtype, label="G=32 FP8 step")


def test_wide_group_edge_semantics():
    """The decode contract holds for wide groups too: a context length outside
    [1, max_context_len] gives NaN rows for that sequence only, and a one-token
    context returns V[0] exactly."""
    from paged_kv_cache_385_amd import decode
    wl = custom_workload([1, 40, 1], 32, 1, 128, dtype="bf16", seed=21)
    cache, segs = build_device(wl)
    out, batch = run_step(wl, cache, segs)
    torch.cuda.synchronize()
    for b in (0, 2):                       # ctx = 1: out = V[0] of the KV head, bit for bit
        _, v = wl.seq_kv(b, segs)
        assert torch.equal(out[b].cpu().view(torch.int16),
                           v[0, 0].expand(32, 128).contiguous().view(torch.int16))
    bad = batch.ctx_d.clone()
    bad[1] = 41                            # beyond max_context_len 40
    d = decode(cache.k_cache, cache.v_cache, wl.q().cuda(), batch.tables_d, bad, 40, wl.scale,
               workspace=batch.workspace)
    torch.cuda.synchronize()
    assert torch.isnan(d[1]).all()
    assert torch.equal(d[0].view(torch.int16), out[0].view(torch.int16))
    assert torch.equal(d[2].view(torch.int16), out[2].view(torch.int16))


def test_wide_group_step_events_time_the_attention():
    """A decode step on a wide group (the several-token kernels, key partitions and their
    merge) with attention events: they are attached to those kernels' dispatches, time a
    positive interval, and leave the output bits as without them."""
    from paged_kv_cache_385_amd import DecodeBatch
    wl = custom_workload([1, 17, 600, 3000], 32, 1, 128, dtype="bf16", seed=7)
    outs = []
    for timed in (False, True):
        cache, segs = build_device(wl)
        batch = DecodeBatch(cache, [op[1] for op in wl.step], wl.num_heads, wl.scale,
                            -(-int(wl.ctx_lens.max()) // 16))
        ks, vs = zip(*(segs.tokens(op[2], op[3], 1) for op in wl.step))
        ev = (torch.cuda.Event(enable_timing=True),
              torch.cuda.Event(enable_timing=True)) if timed else None
        out = batch.step(torch.cat(ks).cuda(), torch.cat(vs).cuda(), wl.q().cuda(),
                         attn_events=ev)
        torch.cuda.synchronize()
        if timed:
            us = ev[0].elapsed_time(ev[1]) * 1e3
            say(f"wide group step: {us:.1f} us between the attention events")
            assert us > 0
        outs.append(out.clone())
        del cache, batch
    assert not torch.isnan(outs[0]).any()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
