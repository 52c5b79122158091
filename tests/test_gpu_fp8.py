"""GPU parity of FP8 (OCP E4M3) pools: quantising writes and copy-on-write copies
bit-exact against the oracle's codes; decode outputs against the oracle's attention
over the dequantised K/V (code * per-head scale), within 2e-3 (float16 q/out) /
1e-2 (bfloat16 q/out)."""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import block_manager as OB
from oracle import cache as OC
from oracle import fp8 as OF
from oracle import layout as OL
from tests.gpu_harness import SegCache, check_close, say
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import paged_kv_cache_385_amd._native as N
    N.lib()


def _scales(wl):
    """Per-KV-head scales; the first head's is small enough that some codes saturate."""
    ks = np.linspace(0.008, 0.03, wl.num_kv_heads).astype(np.float32)
    vs = np.linspace(0.02, 0.006, wl.num_kv_heads).astype(np.float32)
    ks[0] = 0.004
    return ks, vs


def _build(wl, ks, vs):
    from paged_kv_cache_385_amd import PagedKVCache
    segs = SegCache(wl)
    cache = PagedKVCache(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype, "cuda",
                         free_order=wl.free_order, fill_bits=0x7F, kv_scales=(ks, vs))
    cache.apply_trace(wl.setup, segs.tokens)
    return cache, segs


def _step(wl, cache, segs):
    from paged_kv_cache_385_amd import DecodeBatch
    sids = [op[1] for op in wl.step]
    mb = -(-int(wl.ctx_lens.max()) // 16)
    batch = DecodeBatch(cache, sids, wl.num_heads, wl.scale, mb)
    batch.out.fill_(float("nan"))
    ks_, vs_ = zip(*(segs.tokens(op[2], op[3], 1) for op in wl.step))
    out = batch.step(torch.cat(ks_).cuda(), torch.cat(vs_).cuda(), wl.q().cuda())
    torch.cuda.synchronize()
    return out, batch


def _oracle_pools8(wl, segs, ks, vs):
    bm = OB.RefBlockManager(wl.num_blocks, 16, wl.free_order)
    kp, vp = OC.empty_pool8(wl.num_blocks, wl.num_kv_heads, wl.head_dim, fill=0x7F)
    for op in list(wl.setup) + [("step",)]:
        if op[0] == "add":
            bm.add_seq(op[1])
        elif op[0] == "fork":
            bm.fork(op[1], op[2])
        elif op[0] == "append":
            slots, cows = bm.append_tokens(op[1], op[4])
            OC.copy_blocks(kp, vp, cows, inplace=True)
            k, v = segs.tokens(op[2], op[3], op[4])
            OC.cache_write8(kp, vp, k, v, slots, ks, vs, inplace=True)
        else:
            slots, cows = bm.append_batch([s[1] for s in wl.step])
            OC.copy_blocks(kp, vp, cows, inplace=True)
            k, v = zip(*(segs.tokens(s[2], s[3], 1) for s in wl.step))
            OC.cache_write8(kp, vp, torch.cat(k), torch.cat(v), slots, ks, vs, inplace=True)
    return kp, vp


def _oracle_out(wl, segs, ks, vs, seqs):
    def seq_kv(b):
        k, v = wl.seq_kv(b, segs)
        kq = OF.dequantize(OF.quantize(k.float().numpy(), ks[None, :, None]), ks[None, :, None])
        vq = OF.dequantize(OF.quantize(v.float().numpy(), vs[None, :, None]), vs[None, :, None])
        return kq, vq
    return OA.decode_batch(wl.q(), seq_kv, wl.ctx_lens, wl.scale, seqs)


@pytest.mark.parametrize("cfg", [1, 4])
def test_fp8_pools_are_the_oracles_codes(cfg):
    """Set-up trace (with copy-on-write copies for workload 4) and one step."""
    wl = make_workload(cfg)
    ks, vs = _scales(wl)
    say(f"FP8 pools, workload {cfg}")
    cache, segs = _build(wl, ks, vs)
    _step(wl, cache, segs)
    kp, vp = _oracle_pools8(wl, segs, ks, vs)
    kd = OL.k8_to_logical(cache.k_cache.cpu().numpy())
    vd = OL.v8_to_logical(cache.v_cache.cpu().numpy())
    assert np.array_equal(kd, kp) and np.array_equal(vd, vp)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_fp8_step_matches_oracle(cfg):
    wl = make_workload(cfg)
    ks, vs = _scales(wl)
    say(f"FP8 decode step, workload {cfg}")
    cache, segs = _build(wl, ks, vs)
    out, _ = _step(wl, cache, segs)
    ref = _oracle_out(wl, segs, ks, vs, range(wl.num_seqs))
    check_close(out, ref, wl.dtype, label=f"fp8 workload {cfg}")


def test_fp8_long_contexts_merge():
    """Workload 5 (32k-128k contexts): many partitions, the separate merge launch."""
    wl = make_workload(5)
    ks, vs = _scales(wl)
    cache, segs = _build(wl, ks, vs)
    out, _ = _step(wl, cache, segs)
    ref = _oracle_out(wl, segs, ks, vs, range(wl.num_seqs))
    check_close(out, ref, wl.dtype, label="fp8 workload 5")


# ---- pa_chunk_attention on FP8 pools: several new tokens per sequence ----------------

def _chunk_fp8(wl, q_lens, seqs, label):
    """Every sequence holds its ctx_b tokens (set-up trace and step replayed as stores);
    the last q_len_b of them are the queries.  Against the oracle's causal attention
    over the dequantised K/V."""
    from paged_kv_cache_385_amd import chunk_attention
    ks, vs = _scales(wl)
    cache, segs = _build(wl, ks, vs)
    cache.apply_trace(wl.step, segs.tokens)
    sids = [op[1] for op in wl.step]
    tables, ctx_d, max_ctx = cache.tables(sids, -(-int(wl.ctx_lens.max()) // 16))
    q_lens = np.asarray(q_lens, dtype=np.int64)
    q = wl.chunk_q(q_lens)
    starts = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    chunk_attention(cache.k_cache, cache.v_cache, q.cuda(), torch.from_numpy(starts).cuda(),
                    tables, ctx_d, int(q_lens.max()), max_ctx, wl.scale, out=out,
                    scales=cache.scales)
    torch.cuda.synchronize()

    def seq_kv(b):
        k, v = wl.seq_kv(b, segs)
        kq = OF.dequantize(OF.quantize(k.float().numpy(), ks[None, :, None]), ks[None, :, None])
        vq = OF.dequantize(OF.quantize(v.float().numpy(), vs[None, :, None]), vs[None, :, None])
        return kq, vq
    ref = OA.chunk_batch(q, starts, seq_kv, wl.ctx_lens, wl.scale, seqs)
    rows = np.concatenate([np.arange(starts[b], starts[b + 1]) for b in seqs])
    check_close(out, ref, wl.dtype, rows=rows, label=label)


def test_fp8_chunk_speculative_verify_shape():
    """70B-shaped GQA-8 batch on FP8 pools, 6 new tokens per sequence: the narrow kernel,
    three 16-column tiles per workgroup, non-temporal loads, sequences longest first."""
    wl = make_workload(3)
    say("FP8 pools, workload 3, 6 new tokens per sequence")
    seqs = sorted(set([0, 1, int(np.argmax(wl.ctx_lens)), int(np.argmin(wl.ctx_lens))]
                      + list(range(5, 128, 17))))
    _chunk_fp8(wl, np.minimum(6, wl.ctx_lens), seqs, "fp8 verify, workload 3")


@pytest.mark.parametrize("q_lens,H,Hkv,D,dt", [
    ([300, 1024, 40, 1], 16, 2, 128, "bf16"),    # wide kernel (G=8): chunks, a whole prompt
    ([40, 64, 7, 1], 16, 2, 64, "f16"),           # wide kernel at head dim 64
    ([5, 3, 6, 2], 16, 2, 128, "f16"),            # narrow, three tiles, key partitions + merge
    ([12, 10, 9, 11], 8, 2, 64, "bf16"),          # narrow, three tiles at head dim 64
    ([1, 2, 1, 2], 4, 4, 128, "bf16"),            # narrow, one tile (MHA)
    ([4, 3, 2, 1], 16, 2, 128, "f16"),            # narrow, two tiles
    ([8, 5, 3, 1], 8, 2, 64, "bf16"),             # narrow, two tiles at head dim 64 (pairs)
    ([2, 1, 3, 4], 4, 4, 64, "f16"),              # narrow, one tile at head dim 64 (pairs)
])
def test_fp8_chunks(q_lens, H, Hkv, D, dt):
    from workloads import custom_workload
    ctx = [700, 1500, 2100, 33]
    wl = custom_workload(ctx, H, Hkv, D, dtype=dt, seed=H + D + q_lens[0])
    say(f"FP8 pools, chunks {q_lens} over {ctx}, H={H} Hkv={Hkv} D={D} {dt}")
    _chunk_fp8(wl, np.minimum(q_lens, ctx), range(len(ctx)), f"fp8 chunks H={H} D={D}")


def test_fp8_chunks_over_long_contexts():
    """Contexts whose waves walk several runs of 64 block ids (up to 9000 tokens), with
    block counts that leave a wave an odd number of blocks: the narrow kernel on FP8
    pools takes blocks in pairs, so a run's last pair may hold a padding step."""
    from workloads import custom_workload
    ctx = [9000, 4500, 4113, 70]
    wl = custom_workload(ctx, 16, 2, 128, dtype="bf16", seed=91)
    say(f"FP8 pools, chunks [6, 3, 5, 2] over {ctx}, H=16 Hkv=2 D=128 bf16")
    _chunk_fp8(wl, np.minimum([6, 3, 5, 2], ctx), range(len(ctx)), "fp8 chunks, long contexts")


def test_fp8_fused_store_contract():
    """The step's quantising store runs inside the attention pass on FP8 pools too:
    the new tokens' codes are the oracle's, and a slot that is not the sequence's last
    position is not stored and poisons only that sequence (a negative slot stores
    nothing)."""
    from paged_kv_cache_385_amd import alloc_workspace, decode_fused
    from tests.test_gpu_parity import _step_inputs
    from workloads import custom_workload
    wl = custom_workload([20, 37, 600, 9], 8, 2, 128, dtype="bf16", seed=12)
    ks, vs = _scales(wl)
    say("FP8 fused store: codes, mismatched and negative slots")
    cache, segs = _build(wl, ks, vs)
    tab, ctx, slots, k_new, v_new = _step_inputs(wl, segs)
    q = wl.q().cuda()
    mx = int(wl.ctx_lens.max())
    ws = alloc_workspace(wl.num_seqs, wl.num_heads, wl.head_dim, mx)
    kb = OL.k8_to_logical(cache.k_cache.cpu().numpy())
    vb = OL.v8_to_logical(cache.v_cache.cpu().numpy())
    bad = slots.clone()
    bad[1] = slots[1] - 1          # an earlier position of sequence 1: rejected, not stored
    bad[3] = -1                    # not stored
    out = decode_fused(cache.k_cache, cache.v_cache, k_new, v_new, bad, q, tab, ctx, mx, wl.scale,
                       workspace=ws, scales=cache.scales)
    torch.cuda.synchronize()
    assert torch.isnan(out[1].float()).all()
    assert not torch.isnan(out[[0, 2]].float()).any()
    check_close(out, _oracle_out(wl, segs, ks, vs, [0, 2]), wl.dtype, rows=[0, 2],
                label="FP8 fused, valid rows")
    kd = OL.k8_to_logical(cache.k_cache.cpu().numpy())
    vd = OL.v8_to_logical(cache.v_cache.cpu().numpy())
    for pool_d, pool_b in ((kd, kb), (vd, vb)):
        diff = np.argwhere((pool_d != pool_b).any(axis=(1, 3)))
        assert {int(b) * 16 + int(t) for b, t in diff} == {int(slots[0]), int(slots[2])}
    for i in (0, 2):
        s = int(slots[i])
        kq = OF.quantize(k_new[i].float().cpu().numpy(), ks[:, None])
        vq = OF.quantize(v_new[i].float().cpu().numpy(), vs[:, None])
        assert np.array_equal(kd[s // 16, :, s % 16, :], kq) and np.array_equal(vd[s // 16, :, s % 16, :], vq)
