#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV-cache hot path on one MI355X.

Workload: the 70B-shaped GQA-8 decode layer (128 sequences, 64 query heads,
8 KV heads, head_dim 128, bf16 cache, context lengths lognormal with median
1024 clipped to [16, 4096], blocks of 16 tokens placed at random).  One step
is the whole hot path for the batch: the host block manager reserves the next
slot of every sequence and packs the tables into pinned memory, one upload of
them (on a side stream, overlapping the previous step's kernels), the
copy-on-write copy (none arise here), the slot-mapped cache write of the 128
new tokens, the attention pass and the log-sum-exp merge.  Contexts grow by
one token per step, as in real decoding.

Prints one JSON line.  ``value`` is K/V bytes the steps had to read divided
by the wall time of the timed steps (GB/s); ``roofline`` rates the attention
kernel alone, timed with HIP events on its stream on about five of the timed steps
(at most every fifth); ``cpu_baseline``
is the CPU oracle on a bounded sample of the same workload.  Other legs:
``--kv-dtype fp8``, ``--block-size 32``, ``--chunk verify|prefill``, ``--prefix``, ``--swap``.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

EVENT_SAMPLES = 5              # timed steps whose attention pass carries a timing event pair
EVENT_MIN_EVERY = 5            # ... at most one in this many
TIMELINE_STEPS = 5             # steps captured with per-workgroup stamps (--timeline)
TIMELINE_HZ = 100e6            # the kernel's stamps count a constant 100 MHz clock
FLUSH_BYTES = 1 << 30          # written before a flushed step: > 8 x 4 MB L2 + 256 MB Infinity Cache
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published peak
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix-core peak, AMD published (no sparsity)
METRIC = "paged-attn decode KV GB/s read (% of HBM peak); sequence-steps/s"
CSRC = os.path.join(ROOT, "paged_kv_cache_385_amd", "csrc")
# per measured leg: the counter summary file, the kernel source it is stamped with and
# the kernel names that make up one call
TRAFFIC = {
    "decode": (os.path.join(ROOT, "profiles", "decode_attn_traffic_{mode}.json"),
               (os.path.join(CSRC, "pa_kernels.hip"), os.path.join(CSRC, "decode_grouped.hip")),
               ("decode_attn_kernel", "decode_merge_kernel", "decode_group_kernel")),
    "chunk": (os.path.join(ROOT, "profiles", "chunk_attn_traffic_{mode}.json"),
              (os.path.join(CSRC, "chunk_attention.hip"),),
              ("chunk_attn_kernel", "chunk_wide_kernel", "chunk_merge_kernel")),
}
CONTEXT_TEXT = {
    1: "17, 33, 64, 100 tokens",
    2: "uniform in [128, 2048]",
    3: "lognormal median 1024, sigma 1, clipped to [16, 4096]",
    4: "16 prompts x 8 samples: 1024 + U{1..15} shared prefix tokens, U{0..512} private",
    5: "uniform in [32768, 131072]",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, help="workload id (3 = 70B-shaped GQA-8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--staging", choices=("mapped", "upload", "side"), default=None,
                    help="how the step's staged tables reach the kernels: read in place from pinned "
                         "host memory, copied on the step's stream, or copied on a side stream "
                         "(overlapping the previous step); default: the decode batch's own choice "
                         "(in place for batches of at most 16 MiB of K/V, else the side stream)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time budget")
    ap.add_argument("--kv-dtype", choices=("native", "fp8"), default="native",
                    help="KV pools in the workload's 16-bit dtype, or as FP8 (E4M3) codes with "
                         "per-KV-head scales (q and out stay 16-bit)")
    ap.add_argument("--prefix", action="store_true",
                    help="measure prefix-cached admission: 64 requests sharing a 2000-token system "
                         "prompt (host block manager + K/V store + pa_chunk_attention), with the "
                         "same step without prefix caching beside it")
    ap.add_argument("--block-size", type=int, choices=(16, 32), default=16,
                    help="tokens per block of the block manager (32: each block is two "
                         "16-token tiles of the pool; the kernels are the same)")
    ap.add_argument("--swap", action="store_true",
                    help="measure swapping every sequence of the 70B-shaped decode batch out to "
                         "pinned host memory and back (pa_bm_swap_* + pa_swap_blocks)")
    ap.add_argument("--chunk", choices=("verify", "prefill"),
                    help="measure pa_chunk_attention instead of the decode step: 'verify' = the "
                         "70B-shaped batch with 6 new tokens per sequence (HBM-bound), 'prefill' = "
                         "the last 1024-token chunk of four 4096-token prompts (matrix-core bound)")
    ap.add_argument("--flush-steps", type=int, default=10,
                    help="after the timed steps, this many more steps each preceded by a "
                         f"{FLUSH_BYTES >> 20} MiB write that evicts L2 and the Infinity Cache "
                         "(outside the attention events): the flushed roofline fraction")
    ap.add_argument("--timeline", metavar="OUT_JSON",
                    help="load libpa_timeline.so (the decode kernel stamps every workgroup), "
                         f"capture {TIMELINE_STEPS} more single steps after the others and write "
                         "the per-workgroup timeline summary to OUT_JSON")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read probes (the measured read ceiling)")
    ap.add_argument("--no-other-ops", action="store_true",
                    help="skip timing pa_copy_blocks and a bulk pa_cache_write")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (reference for HBM counters)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --copy-calibration MIB' into the per-launch traffic file")
    return ap.parse_args()


def source_sha256(paths) -> str:
    """sha256 of the leg's kernel sources, concatenated in order."""
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_leg(args):
    """(summary file, stamped source, kernel names, workload key) of the measured leg."""
    fp8 = getattr(args, "kv_dtype", "native") == "fp8"
    if args.chunk:
        path, src, names = TRAFFIC["chunk"]
        mode = args.chunk + ("_fp8" if fp8 else "")
        return path.format(mode=mode), src, names, f"chunk-{mode}"
    path, src, names = TRAFFIC["decode"]
    mode = f"w{args.workload}" + ("_fp8" if fp8 else "")
    return path.format(mode=mode), src, names, mode


def summarize_counters(args):
    """Per-call HBM traffic of the measured leg's kernels from two counter runs.

    Each counter is scaled by what it reads for the calibration copy (a plain
    device copy of known size run by the same command): bytes moved / counter.
    The timed calls are the last ``--steps`` ones; a call is every launch of the
    leg's kernels (a chunk call may add a merge launch).
    """
    import csv
    path_out, src, names, key = traffic_leg(args)
    out = {"kernel": None, "workload": key, "steps": args.steps, "warmup": args.warmup,
           "copy_bytes": args.copy_calibration << 20}
    for name, path in (("fetch", args.summarize_counters[0]), ("write", args.summarize_counters[1])):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        attn = [r for r in rows if any(k in r["Kernel_Name"] for k in names)]
        first = int(attn[0]["Dispatch_Id"])
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"] and int(r["Dispatch_Id"]) < first]
        calib = copies[-3:]                       # the three calibration copies come last
        kib = float(np.mean([float(r["Counter_Value"]) for r in calib]))
        scale = out["copy_bytes"] / (kib * 1024.0)
        calls = args.steps + args.warmup + (0 if args.chunk else args.flush_steps)
        per_call = len(attn) // calls
        if per_call < 1 or len(attn) != per_call * calls:
            raise SystemExit(f"{path}: {len(attn)} launches of {names} for {calls} calls: "
                             "run with the --steps, --warmup and --flush-steps of the counter runs")
        timed = attn[args.warmup * per_call:(args.warmup + args.steps) * per_call]
        mean_kib = float(np.sum([float(r["Counter_Value"]) for r in timed])) / args.steps
        out[f"{name}_counter"] = timed[0]["Counter_Name"]
        out[f"{name}_copy_kib"] = kib
        out[f"{name}_scale"] = round(scale, 4)
        out[f"{name}_kib_per_launch"] = round(mean_kib, 1)
        out[f"{name}_bytes_per_launch"] = int(mean_kib * 1024.0 * scale)
        out["kernel"] = " + ".join(sorted({r["Kernel_Name"] for r in timed}))
        out["launches"] = len(timed)
    out["traffic_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    out["source_sha256"] = source_sha256(src)
    with open(path_out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def recorded_traffic(args):
    """The leg's counter summary (traffic per call and the steps and warm-up of the run it
    was taken on), if it was taken on this kernel source and workload; else None."""
    path, src, _, key = traffic_leg(args)
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_sha256(src) or t.get("workload") != key:
        return None
    return t


def traffic_fields(rec, algorithmic_bytes):
    """roofline.traffic and its context: the counter run's HBM bytes per call, that run's
    algorithmic bytes per call (``algorithmic_bytes(steps, warmup)``) and their ratio."""
    if rec is None:
        return {"traffic": None}
    t = int(rec["traffic_bytes_per_launch"])
    alg = algorithmic_bytes(int(rec["steps"]), int(rec["warmup"]))
    return {"traffic": t, "traffic_run": {"steps": rec["steps"], "warmup": rec["warmup"],
                                          "algorithmic_bytes": int(alg),
                                          "fetch_bytes": rec["fetch_bytes_per_launch"],
                                          "write_bytes": rec["write_bytes_per_launch"]},
            "traffic_ratio": round(t / alg, 4)}


def calibration_copy(args, dev):
    """Three device-to-device copies of --copy-calibration MiB, right before the timed
    launches: the counter runs scale FETCH_SIZE and WRITE_SIZE by what they read here."""
    import torch
    if not args.copy_calibration:
        return
    n = args.copy_calibration << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy: 3 x {args.copy_calibration} MiB device-to-device")
    del src, dst


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def blas_threads() -> int:
    """Threads the oracle's numpy products may use (the largest BLAS pool)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return 1


def host_info() -> dict:
    """The host the CPU baseline runs on: logical CPUs, those this process may use, model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_count": os.cpu_count(), "usable_cpus": usable, "model": model,
            "blas_threads": blas_threads()}


def _timed_oracle(wl, budget_s: float, kv_cache: dict):
    """The oracle on the workload's sequences in order until the budget is spent; returns
    (seconds, CPU seconds of the process, K/V bytes, sequences).  Generating a sequence's
    K/V is not timed and happens once: `kv_cache` keeps it for the next cycles."""
    from oracle import attention as OA
    q = wl.q()
    t_total, cpu_total, kv_bytes, seqs = 0.0, 0.0, 0, 0
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * 2
    b = 0
    t_log = time.perf_counter()
    while t_total < budget_s:
        i = b % wl.num_seqs
        if i not in kv_cache:
            kv_cache[i] = wl.seq_kv(i)
        k, v = kv_cache[i]
        if time.perf_counter() - t_log > 20.0:
            log(f"CPU oracle: {seqs} sequences, {t_total:.1f} of {budget_s:.1f} s timed")
            t_log = time.perf_counter()
        c0 = time.process_time()
        t0 = time.perf_counter()
        OA.decode_attention(q[b % wl.num_seqs], k, v, wl.scale)
        t_total += time.perf_counter() - t0
        cpu_total += time.process_time() - c0
        kv_bytes += int(wl.ctx_lens[b % wl.num_seqs]) * per_tok
        seqs += 1
        b += 1
    return t_total, cpu_total, kv_bytes, seqs


def cpu_baseline(wl, budget_s: float):
    """The oracle, as it stands, on the workload's sequences: once with the BLAS pool at
    its default size, once limited to one thread, half the budget each.  ``cores`` is
    the threads the oracle actually kept busy (process CPU time / wall time)."""
    info = host_info()
    kv_cache = {}
    t, c, kvb, n = _timed_oracle(wl, budget_s / 2, kv_cache)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1, c1, kvb1, n1 = _timed_oracle(wl, budget_s / 2, kv_cache)
        one = {"value": kvb1 / t1 / 1e9, "seq_steps_per_s": n1 / t1,
               "cores": round(c1 / t1, 2), "sequences": n1}
    except Exception as e:                       # threadpoolctl missing: report the one run
        log(f"one-thread oracle run skipped: {e}")
    return {"value": kvb / t / 1e9, "unit": "GB/s", "cores": round(c / t, 2),
            "kind": "oracle", "seq_steps_per_s": n / t,
            "threads_allowed": info["blas_threads"], "host": info, "one_thread": one,
            "sample": f"{n} sequence decodes cycling over the workload's {wl.num_seqs} sequences "
                      f"({kvb / 1e6:.1f} MB of K/V) in {t:.1f} s with the BLAS pool at "
                      f"{info['blas_threads']} threads, then the same at 1 thread; float64 numpy"}


def _time_launches(fn, reps: int, stream) -> float:
    """Average microseconds per call of ``reps`` back-to-back calls between one event pair."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()                                       # untimed first call
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def read_ceiling(cache, sids, max_blocks, wl, dev, achieved_gbs, reps: int = 10):
    """Measured read ceilings (pa_probe_read_*): a contiguous 2 GiB read, and a gather of
    exactly the (block, KV head) tiles the decode pass reads, K and V, in a shuffled order
    (the decode pass reads them in its own order), at the pool's tile size (4 KiB for a
    16-bit pool at head dim 128, 2 KiB for an FP8 one).  Each at 2, 4 and 8 workgroups per
    compute unit; the best is reported."""
    import ctypes as C
    import torch
    from paged_kv_cache_385_amd import _native
    lib = _native.lib()
    stream = torch.cuda.current_stream(dev)
    sp = C.c_void_p(stream.cuda_stream)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    buf = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    contiguous = {}
    for wg in (2, 4, 8):
        us = _time_launches(lambda: _native.check(lib.pa_probe_read_contiguous(
            buf.data_ptr(), buf.numel(), wg, sink.data_ptr(), sp), "pa_probe_read_contiguous"),
            reps, stream)
        contiguous[wg] = buf.numel() / (us * 1e-6) / 1e9
    del buf
    tab, ctx = cache.bm.pack(np.asarray(sids, dtype=np.int64), max_blocks)
    Hkv = wl.num_kv_heads
    tiles = np.concatenate([(tab[b, :-(-int(ctx[b]) // 16)].astype(np.int64)[:, None] * Hkv
                             + np.arange(Hkv)[None, :]).ravel() for b in range(len(ctx))])
    tiles = np.random.default_rng(385).permutation(tiles).astype(np.int32)
    tiles_d = torch.from_numpy(tiles).to(dev)
    pool_bytes = cache.k_cache.numel() * cache.k_cache.element_size()
    one_tile = 16 * wl.head_dim * (1 if cache.fp8 else cache.k_cache.element_size())
    tile_bytes = 2 * len(tiles) * one_tile
    gather = {}
    for wg in (2, 4, 8):
        us = _time_launches(lambda: _native.check(lib.pa_probe_read_tiles(
            cache.k_cache.data_ptr(), cache.v_cache.data_ptr(), pool_bytes, one_tile,
            tiles_d.data_ptr(), tiles.ctypes.data, len(tiles), wg, sink.data_ptr(), sp),
            "pa_probe_read_tiles"), reps, stream)
        gather[wg] = tile_bytes / (us * 1e-6) / 1e9
    bc, bg = max(contiguous, key=contiguous.get), max(gather, key=gather.get)
    log(f"read ceiling: contiguous {contiguous[bc]:.0f} GB/s ({bc} workgroups/CU), gather of "
        f"{one_tile}-byte tiles {gather[bg]:.0f} GB/s ({bg} workgroups/CU) over "
        f"{tile_bytes / 1e6:.1f} MB")
    return {"unit": "GB/s", "contiguous": round(contiguous[bc], 1),
            "tile_gather": round(gather[bg], 1),
            "frac_of_tile_gather": round(achieved_gbs / gather[bg], 4),
            "contiguous_bytes": 2 << 30, "tile_gather_bytes": tile_bytes,
            "tile_bytes": one_tile,
            "workgroups_per_cu": {"contiguous": bc, "tile_gather": bg},
            "kernels": "probe_contiguous_kernel, probe_tiles_kernel (pa_probe.h)"}


def other_ops(dev, reps: int = 20):
    """pa_copy_blocks and a bulk pa_cache_write, in GB/s of bytes read + written.
    copy-on-write: the 112 pairs of the shared-prefix workload (16 prompts x 7 copies of
    the partly filled last prefix block; 32 KV heads, head_dim 128, float16: 128 KiB of K
    and 128 KiB of V per block) in one call.  Bulk write: 131072 tokens of the 70B-shaped
    layer (8 KV heads, head_dim 128, bfloat16) into 8192 blocks, 16 consecutive slots per
    block, the blocks in random order (a prefill's store)."""
    import torch
    import paged_kv_cache_385_amd as pa
    stream = torch.cuda.current_stream(dev)
    rng = np.random.default_rng(385)
    out = {}
    nb, hkv, d = 2048, 32, 128
    k, v = pa.alloc_pool(nb, hkv, d, torch.float16, dev, fill_bits=0x3C00)
    perm = rng.permutation(nb)
    pairs_h = np.ascontiguousarray(np.stack([perm[:112], perm[112:224]], 1).astype(np.int32))
    pairs = torch.from_numpy(pairs_h).to(dev)
    us = _time_launches(lambda: pa.copy_blocks(k, v, pairs, pairs_host=pairs_h), reps, stream)
    moved = 2 * 112 * 2 * hkv * 16 * d * 2
    out["copy_blocks"] = {"pairs": 112, "us": round(us, 2), "bytes": moved,
                          "gbs": round(moved / (us * 1e-6) / 1e9, 1),
                          "frac": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                          "kernel": "block_copy_kernel"}
    del k, v, pairs
    nb, hkv, T = 8192, 8, 131072
    k, v = pa.alloc_pool(nb, hkv, d, torch.bfloat16, dev, fill_bits=0)
    blocks = rng.permutation(nb)[:T // 16]
    slots = torch.from_numpy((blocks[:, None] * 16 + np.arange(16)[None, :]).ravel().astype(np.int64)).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(385)
    kn = torch.randn((T, hkv, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    vn = torch.randn((T, hkv, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    us = _time_launches(lambda: pa.cache_write(k, v, kn, vn, slots), reps, stream)
    moved = 2 * T * 2 * hkv * d * 2 + 8 * T
    out["cache_write_bulk"] = {"tokens": T, "us": round(us, 2), "bytes": moved,
                               "gbs": round(moved / (us * 1e-6) / 1e9, 1),
                               "frac": round(moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                               "kernel": "cache_write_kernel"}
    log(f"other ops: copy_blocks 112 pairs {out['copy_blocks']['us']:.1f} us "
        f"({out['copy_blocks']['gbs']:.0f} GB/s); cache_write {T} tokens "
        f"{out['cache_write_bulk']['us']:.1f} us ({out['cache_write_bulk']['gbs']:.0f} GB/s)")
    return out


def chunk_workload(mode):
    """Workload, new tokens per sequence and a name for a pa_chunk_attention measurement."""
    from workloads import custom_workload, make_workload
    if mode == "verify":
        wl = make_workload(3)
        return (wl, np.minimum(6, wl.ctx_lens), "70B-shaped GQA-8 speculative verify, 6 new tokens "
                "per sequence, B=128, lognormal contexts")
    wl = custom_workload([4096] * 4, 64, 8, 128, dtype="bf16", seed=385)
    return (wl, np.full(4, 1024), "70B-shaped GQA-8 prefill, last 1024-token chunk of four "
            "4096-token prompts")


def chunk_flops(ctx, q_lens, num_heads, head_dim) -> int:
    """Matrix flops of the causal chunk: 2 products x 2 flops per multiply-add per visible key."""
    total = 0
    for c, n in zip(ctx, q_lens):
        visible = np.arange(int(c) - int(n), int(c)) + 1
        total += int(visible.sum()) * 4 * num_heads * head_dim
    return total


def run_chunk(args):
    import torch
    from oracle import attention as OA
    import paged_kv_cache_385_amd as pa
    from paged_kv_cache_385_amd import _native
    assert torch.cuda.is_available(), "no HIP device"
    _native.lib()
    dev = torch.device("cuda:0")
    wl, q_lens, name = chunk_workload(args.chunk)
    B, H, Hkv, D = wl.num_seqs, wl.num_heads, wl.num_kv_heads, wl.head_dim
    K, W = args.steps, args.warmup
    log(f"chunk {args.chunk}: {name}; total new tokens {int(q_lens.sum())}")
    t0 = time.perf_counter()
    fp8 = args.kv_dtype == "fp8"
    kv_scales = (np.full(Hkv, 0.0125, np.float32), np.full(Hkv, 0.0125, np.float32)) if fp8 else None
    cache = pa.PagedKVCache(wl.num_blocks, Hkv, D, wl.dtype, dev, free_order=wl.free_order,
                            kv_scales=kv_scales)
    segs = {}

    def tokens(seg, start, n):
        if seg not in segs:
            segs[seg] = wl.segment_kv(seg)
        k, v = segs[seg]
        return k[start:start + n].contiguous(), v[start:start + n].contiguous()

    cache.apply_trace(wl.setup, tokens)
    cache.apply_trace(wl.step, tokens)            # every sequence now holds ctx_b tokens
    segs.clear()
    sids = [op[1] for op in wl.step]
    max_blocks = -(-int(wl.ctx_lens.max()) // 16)
    tables, ctx_d, max_ctx = cache.tables(sids, max_blocks)
    q = wl.chunk_q(q_lens).to(dev)
    starts = torch.from_numpy(np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)).to(dev)
    out = torch.empty_like(q)
    mq = int(q_lens.max())
    need = pa.chunk_workspace_size(B, H, Hkv, D, int(q_lens.sum()), mq, max_ctx)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"set-up {time.perf_counter() - t0:.1f} s; workspace {need} bytes "
        f"({'key partitions + merge launch' if need else 'one partition'})")
    stream = torch.cuda.current_stream(dev)
    calibration_copy(args, dev)

    def call(events=None):
        pa.chunk_attention(cache.k_cache, cache.v_cache, q, starts, tables, ctx_d, mq, max_ctx,
                           wl.scale, out=out, workspace=ws if need else None, scales=cache.scales,
                           events=events)

    for _ in range(W):
        call()
    # each call's events are attached to its dispatches: start of the attention kernel,
    # end of the call's last kernel (the kernels' own time, as the profiler sees it)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for a, b in ev:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for pair in ev:
        call(pair)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    per_tok = 2 * Hkv * D * (1 if fp8 else 2)     # K and V bytes per cached token
    kv_bytes = int(wl.ctx_lens.sum()) * per_tok
    io_bytes = 2 * int(q_lens.sum()) * H * D * 2 + int((-(-wl.ctx_lens // 16)).sum()) * 4 + 8 * B
    flops = chunk_flops(wl.ctx_lens, q_lens, H, D)
    log(f"{K} calls: wall {wall * 1e3:.2f} ms ({wall * 1e6 / K:.1f} us per call), kernels "
        f"{us:.1f} us per call (events on the dispatches)")
    if args.chunk == "verify":
        metric, unit = "paged-attn verify KV GB/s read (% of HBM peak)", "GB/s"
        value = (kv_bytes + io_bytes) / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(value / HBM_PEAK_GBS, 4)}
    else:
        metric, unit = "paged-attn prefill-chunk TFLOP/s (% of bf16 matrix peak)", "TFLOP/s"
        value = flops / (us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(value, 1), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(value / MFMA_BF16_PEAK_TFS, 4)}
    kname = "chunk_wide_kernel" if mq * (H // Hkv) >= 128 else "chunk_attn_kernel"
    roof.update(traffic_fields(recorded_traffic(args), lambda s_, w_: kv_bytes + io_bytes))
    roof.update({"kernel": f"{kname}<{wl.dtype_name.upper()},{D}" + (",FP8>" if fp8 else ">")
                 + (" + chunk_merge_kernel" if need else ""),
                 "avg_launch_us": round(us, 2), "bytes_per_launch": kv_bytes + io_bytes,
                 "flops_per_launch": flops})
    result = {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": K,
              "warmup": W, "ms_per_step": round(wall * 1e3 / K, 4), "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype_name, "data": "synthetic",
              "config": {"workload": name, "batch": B, "num_heads": H, "num_kv_heads": Hkv,
                         "head_dim": D, "block_size": 16,
                         "kv_dtype": "fp8_e4m3" if fp8 else wl.dtype_name,
                         "new_tokens": int(q_lens.sum()), "max_new_tokens": mq,
                         "mean_context": round(float(wl.ctx_lens.mean()), 1)},
              "roofline": roof}
    if not args.no_cpu_baseline:
        log("CPU oracle baseline ...")
        qc = wl.chunk_q(q_lens)
        st = np.concatenate([[0], np.cumsum(q_lens)])
        t_total, c_total, done_b, done_f = 0.0, 0.0, 0, 0
        b = 0
        while t_total < args.cpu_seconds and b < 4 * B:
            bb = b % B
            k, v = wl.seq_kv(bb)
            n = int(q_lens[bb])
            rows = slice(int(st[bb]), int(st[bb]) + n)
            c1 = time.process_time()
            t1 = time.perf_counter()
            OA.chunk_attention(qc[rows], k, v, wl.scale)
            t_total += time.perf_counter() - t1
            c_total += time.process_time() - c1
            done_b += int(wl.ctx_lens[bb]) * per_tok
            done_f += chunk_flops([wl.ctx_lens[bb]], [n], H, D)
            b += 1
        cpu = done_b / t_total / 1e9 if unit == "GB/s" else done_f / t_total / 1e12
        result["cpu_baseline"] = {"value": cpu, "unit": unit, "cores": round(c_total / t_total, 2),
                                  "kind": "oracle", "host": host_info(),
                                  "sample": f"{b} sequences' chunks, float64 numpy, {t_total:.1f} s"}
    print(json.dumps(result), flush=True)


PREFIX_REQUESTS = 64
PREFIX_SYSTEM = 2000
PREFIX_QUERY = (16, 128)


def run_prefix(args):
    """Admission of a batch of requests that share a system prompt, with and without
    prefix caching.  One step: host admission (match, slots, commit of the ids), the
    store of the computed tokens' K/V, and pa_chunk_attention of those tokens over the
    whole context; then every sequence ends.  Each step brings fresh private queries,
    so only the system prompt is reused (its blocks stay cached between steps)."""
    import torch
    import paged_kv_cache_385_amd as pa
    from paged_kv_cache_385_amd import _native
    from paged_kv_cache_385_amd.block_manager import BlockManager
    from workloads.prefix import prompt_ids
    assert torch.cuda.is_available(), "no HIP device"
    _native.lib()
    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    B, H, Hkv, D, dt = PREFIX_REQUESTS, 64, 8, 128, torch.bfloat16
    name = (f"70B-shaped GQA-8 layer, {B} requests sharing a {PREFIX_SYSTEM}-token system prompt, "
            f"private queries U{{{PREFIX_QUERY[0]}..{PREFIX_QUERY[1]}}} tokens")
    log(f"prefix: {name}")
    system = prompt_ids(385, 0, PREFIX_SYSTEM)
    qrng = np.random.default_rng(np.random.SeedSequence([385, 99]))
    # token ids as int32 arrays, the form a tokenizer hands over
    steps_prompts = [[np.asarray(system + prompt_ids(385, 1 + s * B + i,
                                                     int(qrng.integers(PREFIX_QUERY[0],
                                                                       PREFIX_QUERY[1] + 1))),
                                 dtype=np.int32)
                      for i in range(B)] for s in range(K + W)]
    flat = [np.concatenate(ps) for ps in steps_prompts]
    offsets = [np.concatenate([[0], np.cumsum([len(p) for p in ps])]).astype(np.int64)
               for ps in steps_prompts]
    longest = max(len(p) for ps in steps_prompts for p in ps)
    max_blocks = -(-longest // 16)
    nb = B * (max_blocks + 1) + 64
    k_cache, v_cache = pa.alloc_pool(nb, Hkv, D, dt, dev, fill_bits=0)
    scale = D ** -0.5
    tmax = B * longest
    g = torch.Generator(device=dev)
    g.manual_seed(385)
    k_all = torch.randn((tmax, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(dt)
    v_all = torch.randn((tmax, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(dt)
    q_all = torch.randn((tmax, H, D), generator=g, device=dev, dtype=torch.float32).to(dt)
    ws_bytes = pa.chunk_workspace_size(B, H, Hkv, D, tmax, longest, longest)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out_all = torch.empty_like(q_all)
    stream = torch.cuda.current_stream(dev)

    # per-step pinned staging (never reused within a run), so the host admission of one
    # step overlaps the kernels of the previous one
    def pinned(shape, dtype):
        return torch.empty(shape, dtype=dtype, pin_memory=True)

    def run(cached_on):
        bm = BlockManager(nb, prefix_caching=cached_on)
        stage = [(pinned(tmax, torch.int64), pinned((B, max_blocks), torch.int32),
                  pinned(B, torch.int32), pinned(B + 1, torch.int32)) for _ in range(K + W)]
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        host_s, shapes = 0.0, []
        sids = np.arange(B, dtype=np.int64)
        torch.cuda.synchronize()
        t_start = None
        for s in range(K + W):
            if s == W:
                torch.cuda.synchronize()
                t_start = time.perf_counter()
                st0 = bm.prefix_stats() if cached_on else None
            prompts = steps_prompts[s]
            th = time.perf_counter()
            h_slots, h_tab, h_ctx, h_starts = stage[s]
            slots = h_slots.numpy()
            if cached_on:                        # one call: match, slots, commit of the ids
                c, sl, _ = bm.admit_batch(sids, flat[s], offsets[s], slots_out=slots)
                new = (np.diff(offsets[s]) - c).tolist()
                pos = sl.shape[0]
            else:
                new, pos = [], 0
                for i, p in enumerate(prompts):
                    bm.add_seq(i)
                    sl, _ = bm.append_tokens(i, len(p))
                    slots[pos:pos + len(p)] = sl
                    pos += len(p)
                    new.append(len(p))
            tables, ctx = bm.pack(sids, max_blocks, tables_out=h_tab.numpy(),
                                  ctx_out=h_ctx.numpy())
            starts = h_starts.numpy()
            starts[0] = 0
            np.cumsum(new, out=starts[1:])
            T = pos
            slots_d = h_slots[:T].to(dev, non_blocking=True)
            tables_d = h_tab.to(dev, non_blocking=True)
            ctx_d = h_ctx.to(dev, non_blocking=True)
            starts_d = h_starts.to(dev, non_blocking=True)
            mq, mc = max(new), int(ctx.max())
            if s >= W:
                host_s += time.perf_counter() - th
                shapes.append((ctx.copy(), list(new)))
            e = ev[s - W] if s >= W else None
            if e:
                e[0].record(stream)
            pa.ops.cache_write(k_cache, v_cache, k_all[:T], v_all[:T], slots_d)
            if e:
                e[1].record(stream)
            pa.chunk_attention(k_cache, v_cache, q_all[:T], starts_d, tables_d, ctx_d, mq, mc,
                               scale, out=out_all[:T], workspace=ws)
            if e:
                e[2].record(stream)
            for i in range(B):
                bm.free_seq(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        write_us = float(np.mean([a.elapsed_time(b) for a, b, _ in ev])) * 1e3
        attn_us = float(np.mean([b.elapsed_time(c) for _, b, c in ev])) * 1e3
        r = {"wall_s": wall, "host_us_per_request": host_s / (K * B) * 1e6,
             "write_us": write_us, "attn_us": attn_us,
             "new_tokens": sum(sum(n) for _, n in shapes) / K,
             "flops": sum(chunk_flops(c, n, H, D) for c, n in shapes) / K}
        if cached_on:
            st = bm.prefix_stats()
            r["hit_rate"] = (st["hit_blocks"] - st0["hit_blocks"]) / max(1, st["query_blocks"] - st0["query_blocks"])
            r["stats"] = st
        return r

    cached = run(True)
    full = run(False)
    for tag, r in (("prefix caching", cached), ("no prefix caching", full)):
        log(f"{tag}: {K} steps, wall {r['wall_s'] * 1e3 / K:.3f} ms/step, host "
            f"{r['host_us_per_request']:.1f} us/request, K/V store {r['write_us']:.1f} us, "
            f"attention {r['attn_us']:.1f} us, {r['new_tokens']:.0f} tokens computed per step")
    value = B * K / cached["wall_s"]
    tfs = cached["flops"] / (cached["attn_us"] * 1e-6) / 1e12
    result = {"metric": "prefix-cached admission requests/s (shared system prompt)",
              "value": round(value, 1), "unit": "requests/s", "n_gpus": 1, "steps": K, "warmup": W,
              "ms_per_step": round(cached["wall_s"] * 1e3 / K, 4), "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
              "config": {"workload": name, "batch": B, "num_heads": H, "num_kv_heads": Hkv,
                         "head_dim": D, "block_size": 16, "kv_dtype": "bf16",
                         "system_prompt": PREFIX_SYSTEM, "query_tokens": list(PREFIX_QUERY)},
              "hit_rate": round(cached["hit_rate"], 4),
              "tokens_computed_per_step": round(cached["new_tokens"], 1),
              "host_us_per_request": round(cached["host_us_per_request"], 2),
              "uncached": {"requests_per_s": round(B * K / full["wall_s"], 1),
                           "ms_per_step": round(full["wall_s"] * 1e3 / K, 4),
                           "tokens_computed_per_step": round(full["new_tokens"], 1),
                           "attn_us": round(full["attn_us"], 1),
                           "write_us": round(full["write_us"], 1)},
              "speedup": round(full["wall_s"] / cached["wall_s"], 2),
              "roofline": {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS,
                           "unit": "TFLOP/s", "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                           "traffic": None, "kernel": "chunk_wide_kernel<BF16,128>",
                           "write_us": round(cached["write_us"], 1),
                           "avg_launch_us": round(cached["attn_us"], 2),
                           "flops_per_launch": int(cached["flops"])}}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefix_cpu_baseline(args, steps_prompts[0], H, Hkv, D, scale)
    print(json.dumps(result), flush=True)


def prefix_cpu_baseline(args, prompts, H, Hkv, D, scale):
    """The oracle on a sample of the same step: its prefix cache admits the requests, and
    its attention computes each admitted request's new tokens (float64 numpy)."""
    from oracle import attention as OA
    from oracle.prefix_cache import RefPrefixCache
    B = len(prompts)
    nb = B * (-(-max(len(p) for p in prompts) // 16) + 1)
    ref = RefPrefixCache(nb)
    rng = np.random.default_rng(7)
    t_total, c_total, done = 0.0, 0.0, 0
    # warm the cache with the first request (not timed), as the timed steps find it warm
    c = ref.add_seq_cached(-1, prompts[0])
    ref.append_tokens(-1, len(prompts[0]) - c)
    ref.commit_tokens(-1, prompts[0][c:])
    ref.free_seq(-1)
    for i, p in enumerate(prompts):
        if t_total > args.cpu_seconds:
            break
        k = rng.standard_normal((len(p), Hkv, D)).astype(np.float32)
        v = rng.standard_normal((len(p), Hkv, D)).astype(np.float32)
        c0 = time.process_time()
        t0 = time.perf_counter()
        c = ref.add_seq_cached(i, p)
        ref.append_tokens(i, len(p) - c)
        ref.commit_tokens(i, p[c:])
        q = rng.standard_normal((len(p) - c, H, D)).astype(np.float32)
        OA.chunk_attention(q, k, v, scale)
        t_total += time.perf_counter() - t0
        c_total += time.process_time() - c0
        done += 1
    return {"value": done / t_total, "unit": "requests/s", "cores": round(c_total / t_total, 2),
            "kind": "oracle", "host": host_info(),
            "sample": f"{done} of the step's {B} requests: oracle prefix-cache admission and "
                      f"float64 attention of their new tokens, {t_total:.1f} s"}


HOST_LINK_PEAK_GBS = 64.0      # PCIe 5.0 x16, one direction, theoretical


def run_swap(args):
    """Swap-out then swap-in of every sequence of a decode batch per step: host block
    manager calls, the pairs' upload and one pa_swap_blocks launch per direction."""
    import torch
    from workloads import make_workload
    import paged_kv_cache_385_amd as pa
    from paged_kv_cache_385_amd import _native
    assert torch.cuda.is_available(), "no HIP device"
    _native.lib()
    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    wl = make_workload(args.workload)
    B, Hkv, D = wl.num_seqs, wl.num_kv_heads, wl.head_dim
    log(f"swap: workload {wl.cfg_id} ({wl.name}), {B} sequences, pool {wl.num_blocks} blocks")
    t0 = time.perf_counter()
    cache = pa.PagedKVCache(wl.num_blocks, Hkv, D, wl.dtype, dev, free_order=wl.free_order,
                            host_blocks=wl.num_blocks)
    segs = {}

    def tokens(seg, start, n):
        if seg not in segs:
            segs[seg] = wl.segment_kv(seg)
        k, v = segs[seg]
        return k[start:start + n].contiguous(), v[start:start + n].contiguous()

    cache.apply_trace(wl.setup, tokens)
    segs.clear()
    sids = [op[1] for op in wl.step]
    torch.cuda.synchronize()
    log(f"set-up {time.perf_counter() - t0:.1f} s")
    stream = torch.cuda.current_stream(dev)
    block_bytes = 2 * Hkv * 16 * D * 2
    ev = []
    n_out = n_in = 0
    for it in range(K + W):
        if it == W:
            torch.cuda.synchronize()
            t_wall = time.perf_counter()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        po = cache.bm.swap_out(sids)                 # host: the pairs to copy
        po_d = torch.from_numpy(po).to(dev)
        e[0].record(stream)
        pa.ops.swap_blocks(cache.k_cache, cache.v_cache, cache.k_host, cache.v_host,
                           _native.PA_SWAP_OUT, po_d, pairs_host=po)
        e[1].record(stream)
        pi = cache.bm.swap_in(sids)
        pi_d = torch.from_numpy(pi).to(dev)
        e[2].record(stream)
        pa.ops.swap_blocks(cache.k_cache, cache.v_cache, cache.k_host, cache.v_host,
                           _native.PA_SWAP_IN, pi_d, pairs_host=pi)
        e[3].record(stream)
        if it >= W:
            ev.append(e)
            n_out, n_in = len(po), len(pi)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    out_us = float(np.mean([a.elapsed_time(b) for a, b, _, _ in ev])) * 1e3
    in_us = float(np.mean([c.elapsed_time(d) for _, _, c, d in ev])) * 1e3
    out_gbs = n_out * block_bytes / (out_us * 1e-6) / 1e9
    in_gbs = n_in * block_bytes / (in_us * 1e-6) / 1e9
    total = (n_out + n_in) * block_bytes
    value = total / (wall / K) / 1e9
    log(f"{K} round trips: {n_out} blocks out, {n_in} in ({n_out * block_bytes / 1e6:.1f} MB each "
        f"way); out {out_us:.0f} us ({out_gbs:.1f} GB/s), in {in_us:.0f} us ({in_gbs:.1f} GB/s), "
        f"wall {wall * 1e3 / K:.2f} ms per round trip")
    result = {"metric": "KV swap GB/s over the host link (out + in, whole round trip)",
              "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
              "ms_per_step": round(wall * 1e3 / K, 4), "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": wl.dtype_name, "data": "synthetic",
              "config": {"workload": f"swap of every sequence of the {wl.name}", "batch": B,
                         "num_kv_heads": Hkv, "head_dim": D, "block_size": 16,
                         "kv_dtype": wl.dtype_name, "blocks_each_way": n_out,
                         "block_bytes": block_bytes},
              "out_gbs": round(out_gbs, 2), "in_gbs": round(in_gbs, 2),
              "roofline": {"bound": "host-link", "achieved": round(max(out_gbs, in_gbs), 2),
                           "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                           "frac": round(max(out_gbs, in_gbs) / HOST_LINK_PEAK_GBS, 4),
                           "traffic": None, "kernel": "block_copy_kernel",
                           "avg_launch_us": round((out_us + in_us) / 2, 2),
                           "bytes_per_launch": n_out * block_bytes}}
    print(json.dumps(result), flush=True)


def timeline_summary(recs, event_us):
    """Summary of one decode launch's per-workgroup records (pa_timeline.h layout): the
    span of the pass, how many workgroups run at once, each one's fixed start-up (item
    known, first tile computed), wave 0's pace per tile, and where the workgroups ran."""
    block = np.nonzero(recs[:, 0] != 0)[0]           # blockIdx.x of every written record
    recs = recs[block]
    t0 = recs[:, 0].min()
    entry, plan, first, loop, out = ((recs[:, i] - t0).astype(np.float64) * (1e6 / TIMELINE_HZ)
                                     for i in range(5))
    has_first = recs[:, 2] != 0
    first = np.where(has_first, first, np.nan)
    tiles = (recs[:, 6] & 0xFFFF).astype(np.int64)
    nw0 = ((recs[:, 6] >> 16) & 0xFFFF).astype(np.int64)
    xcc = (recs[:, 7] >> 32).astype(np.int64)
    hw = (recs[:, 7] & 0xFFFFFFFF).astype(np.int64)
    # a compute unit: XCC, shader engine (HW_ID bits 15:13), array (bit 12), CU (bits 11:8)
    cu = (xcc << 8) | (((hw >> 13) & 0x7) << 5) | (((hw >> 12) & 0x1) << 4) | ((hw >> 8) & 0xF)
    # workgroups running over time: +1 at entry, -1 once the output is written
    ev = np.concatenate([np.stack([entry, np.ones_like(entry)], 1),
                         np.stack([out, -np.ones_like(out)], 1)])
    ev = ev[np.lexsort((ev[:, 1], ev[:, 0]))]
    active = np.cumsum(ev[:, 1])
    span = float(out.max())
    edges = np.arange(0.0, span + 10.0, 10.0)

    def pct(x, q):
        return round(float(np.nanpercentile(x, q)), 2)

    startup = first - entry
    late = np.argsort(entry)[-256:]                  # the last 256 workgroups to start
    # the workgroups resident from the start (entered before any workgroup finished), per
    # compute unit in block order: the start-up of the CU's 1st, 2nd, ... of them
    initial = entry < out.min()
    by_rank = {}
    for c in np.unique(cu[initial]):
        idx = np.nonzero(initial & (cu == c))[0]
        for rank, i in enumerate(idx[np.argsort(block[idx])]):
            by_rank.setdefault(rank, []).append(startup[i])
    paced = has_first & (nw0 >= 4)
    pace = (loop - first)[paced] / (nw0[paced] - 1)
    r = recs.astype(np.int64)
    ordered = ((r[:, 0] <= r[:, 1]) & (r[:, 1] <= r[:, 3]) & (r[:, 3] <= r[:, 4]) &
               ((r[:, 2] == 0) | ((r[:, 1] <= r[:, 2]) & (r[:, 2] <= r[:, 3]))))
    return {
        "workgroups": int(len(recs)),
        "misordered": int((~ordered).sum()),
        "tiles_per_kv_head": int(tiles.sum()),
        "span_us": round(span, 2),
        "event_us": round(event_us, 2),
        "max_running": int(active.max()),
        "max_running_reached_us": round(float(ev[np.argmax(active), 0]), 2),
        "running_per_10us": [int(((entry < hi) & (out > lo)).sum())
                             for lo, hi in zip(edges[:-1], edges[1:])],
        "plan_us": {"median": pct(plan - entry, 50), "p90": pct(plan - entry, 90)},
        "first_tile_after_plan_us": {"median": pct(first - plan, 50), "p90": pct(first - plan, 90)},
        "startup_us": {"median": pct(startup, 50), "p90": pct(startup, 90)},
        "initial_per_cu": int(initial.sum()) / max(len(np.unique(cu[initial])), 1),
        "initial_startup_by_block_rank_us": [
            {"median": pct(np.array(v), 50), "p90": pct(np.array(v), 90)}
            for _, v in sorted(by_rank.items())],
        "last_256_start_us": [round(float(entry[late].min()), 2), round(float(entry[late].max()), 2)],
        "last_256_startup_us": {"median": pct(startup[late], 50), "p90": pct(startup[late], 90)},
        "wave0_us_per_tile": {"median": pct(pace, 50), "p10": pct(pace, 10), "p90": pct(pace, 90)},
        "per_xcc": [int((xcc == x).sum()) for x in range(8)],
        # blocks whose index leaves residue r mod 8: the XCCs they ran on (one each when
        # the dispatcher deals blocks to the XCDs in turn)
        "xcc_of_block_mod_8": [sorted(int(x) for x in np.unique(xcc[block % 8 == m]))
                               for m in range(8)],
        "compute_units": int(len(np.unique(cu))),
    }


def capture_timeline(path, native, batch, steps_kv, q, wl, first_step):
    """Single decode steps with the instrumented library: clear the records, run the
    step (attention pass between events), read every workgroup's record; the summaries
    go to `path` as JSON."""
    import torch
    lib = native.lib()
    recs = np.zeros((native.TIMELINE_MAX_WORKGROUPS, native.TIMELINE_WORDS), dtype=np.uint64)
    launches, raw, blocks = [], [], []
    for i, (k, v) in enumerate(steps_kv):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        native.check(lib.pa_timeline_clear(batch.stream.cuda_stream), "pa_timeline_clear")
        batch.step(k, v, q, attn_events=(e0, e1))
        torch.cuda.synchronize()
        native.check(lib.pa_timeline_read(recs.ctypes.data, recs.shape[0]), "pa_timeline_read")
        if batch.last_grouped or not (recs[:, 0] != 0).any():
            raise SystemExit("--timeline: the step ran no decode_attn_kernel (grouped decode and "
                             "the chunk kernels take no stamps)")
        t = {"step": first_step + i, **timeline_summary(recs, e0.elapsed_time(e1) * 1e3)}
        launches.append(t)
        log(f"timeline: {t['workgroups']} workgroups, span {t['span_us']} us (events "
            f"{t['event_us']} us), at most {t['max_running']} running "
            f"(reached at {t['max_running_reached_us']} us), start-up median "
            f"{t['startup_us']['median']} p90 {t['startup_us']['p90']} us, wave 0 "
            f"{t['wave0_us_per_tile']['median']} us per tile, {t['compute_units']} CUs, "
            f"XCC of block mod 8: {t['xcc_of_block_mod_8']}")
        raw.append(recs[recs[:, 0] != 0].copy())
        blocks.append(np.nonzero(recs[:, 0] != 0)[0])
    with open(path, "w") as f:
        json.dump({"workload": wl.cfg_id, "name": wl.name, "library": "libpa_timeline.so",
                   "clock_hz": TIMELINE_HZ, "launches": launches}, f, indent=1)
        f.write("\n")
    # the raw records beside it: records_i (pa_timeline.h layout) and blocks_i (blockIdx.x)
    np.savez_compressed(os.path.splitext(path)[0] + "_records.npz",
                        **{f"records_{i}": r for i, r in enumerate(raw)},
                        **{f"blocks_{i}": b for i, b in enumerate(blocks)})


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.timeline and (args.swap or args.prefix or args.chunk):
        print("--timeline stamps the decode kernel: not with --swap, --prefix or --chunk",
              file=sys.stderr)
        sys.exit(2)
    if args.swap:
        if args.gpus != 1:
            print(f"bench.py measures one GPU only (asked for --gpus {args.gpus})", file=sys.stderr)
            sys.exit(2)
        run_swap(args)
        return
    if args.prefix:
        if args.gpus != 1:
            print(f"bench.py measures one GPU only (asked for --gpus {args.gpus})", file=sys.stderr)
            sys.exit(2)
        run_prefix(args)
        return
    if args.chunk:
        if args.gpus != 1:
            print(f"bench.py measures one GPU only (asked for --gpus {args.gpus})", file=sys.stderr)
            sys.exit(2)
        run_chunk(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.timeline:
        # the instrumented build of the same library (before the binding loads one)
        os.environ["PA_LIB_PATH"] = os.path.join(ROOT, "paged_kv_cache_385_amd", "libpa_timeline.so")
    import torch
    from workloads import make_workload, new_token_kv
    import paged_kv_cache_385_amd as pa
    from paged_kv_cache_385_amd import _native

    assert torch.cuda.is_available(), "no HIP device"
    _native.lib()
    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    F = args.flush_steps
    T = TIMELINE_STEPS if args.timeline else 0
    wl = make_workload(args.workload, grow=K + W + F + T)
    B, H, Hkv, D = wl.num_seqs, wl.num_heads, wl.num_kv_heads, wl.head_dim
    log(f"workload {wl.cfg_id} ({wl.name}): B={B} H={H} Hkv={Hkv} D={D} {wl.dtype_name}, "
        f"ctx mean {wl.ctx_lens.mean():.0f} max {wl.ctx_lens.max()}, pool {wl.num_blocks} blocks")

    # ---- set-up (not timed): replay the history through the library ----
    t0 = time.perf_counter()
    fp8 = args.kv_dtype == "fp8"
    # FP8 scales: the synthetic K/V are standard normal, so |x| / 0.0125 reaches the
    # E4M3 range (448) only past 5.6 sigma
    kv_scales = (np.full(Hkv, 0.0125, np.float32), np.full(Hkv, 0.0125, np.float32)) if fp8 else None
    if args.block_size == 16:
        cache = pa.PagedKVCache(wl.num_blocks, Hkv, D, wl.dtype, dev, free_order=wl.free_order,
                                kv_scales=kv_scales)
    else:   # 32-token blocks waste up to 31 tokens per sequence: a larger pool of tile pairs
        tiles = 2 * -(-int(1.25 * wl.num_blocks) // 2)
        cache = pa.PagedKVCache(tiles, Hkv, D, wl.dtype, dev, kv_scales=kv_scales, block_size=32)
    segs = {}

    def tokens(seg, start, n):
        if seg not in segs:
            segs[seg] = wl.segment_kv(seg)
        k, v = segs[seg]
        return k[start:start + n].contiguous(), v[start:start + n].contiguous()

    cache.apply_trace(wl.setup, tokens)
    segs.clear()
    sids = [op[1] for op in wl.step]
    bsz = args.block_size
    max_blocks = -(-(int(wl.ctx_lens.max()) + K + W + F + T) // bsz) * (bsz // 16)   # 16-token tiles
    batch = pa.DecodeBatch(cache, sids, H, wl.scale, max_blocks, staging=args.staging)
    q = wl.q().to(dev)
    steps_kv = []
    for i in range(K + W + F + T):
        k, v = new_token_kv(wl.seed, i, B, Hkv, D, wl.dtype)
        steps_kv.append((k.to(dev), v.to(dev)))
    torch.cuda.synchronize()
    log(f"set-up {time.perf_counter() - t0:.1f} s")

    calibration_copy(args, dev)

    per_tok = 2 * Hkv * D * (1 if fp8 else 2)     # K and V bytes per cached token
    base_ctx = wl.ctx_lens.astype(np.int64)

    def step_bytes(i):   # algorithmic bytes of the attention pass at step i (0-based)
        ctx = base_ctx + i
        blocks = -(-ctx // 16)
        return int(ctx.sum()) * per_tok + 2 * B * H * D * 2 + int(blocks.sum()) * 4 + 4 * B

    for i in range(W):
        batch.step(*steps_kv[i], q)
    torch.cuda.synchronize()

    # The attention pass is timed with events on about EVENT_SAMPLES steps spread over the
    # timed ones (every `every`-th): events attached to a dispatch delay the next kernel by
    # about 9 us, which is charged to the step.  Timing events are created (first record)
    # before the timed region.
    every = max(EVENT_MIN_EVERY, K // EVENT_SAMPLES)
    sampled = [j for j in range(K) if j % every == 0]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sampled]
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(F)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for e in [start, stop] + [x for pair in ev + fev for x in pair]:
        e.record(batch.stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(batch.stream)
    for j in range(K):
        batch.step(*steps_kv[W + j], q,
                   attn_events=ev[j // every] if j % every == 0 else None)
    stop.record(batch.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    gpu_ms = start.elapsed_time(stop)
    attn_ms = [a.elapsed_time(b) for a, b in ev]

    # Flushed variant (after the timed region): before each of F more steps, a write of
    # FLUSH_BYTES evicts the pools from L2 and the Infinity Cache, outside the events.
    flushed_ms = []
    if F:
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        for j in range(F):
            flush.fill_(j & 0xFF)
            batch.step(*steps_kv[W + K + j], q, attn_events=fev[j])
        torch.cuda.synchronize()
        flushed_ms = [a.elapsed_time(b) for a, b in fev]
        del flush

    if T:
        capture_timeline(args.timeline, _native, batch, steps_kv[W + K + F:], q, wl, W + K + F)

    kv_read = sum(int((base_ctx + W + j).sum()) * per_tok for j in range(K))
    value = kv_read / wall / 1e9
    attn_avg_ms = float(np.mean(attn_ms))
    # HBM minimum: every distinct cached token once.  The block manager counts, per used
    # block, the most tokens any sharer keeps in it; all live sequences are the batch's,
    # and each step adds one private token per sequence.
    occupied = int(cache.bm.stats()["occupied_slots"])
    last = W + K + F + T - 1                   # the step the block manager's count is taken at

    def unique_bytes(i):
        ctx = base_ctx + i
        tokens = occupied - B * (last - i)
        return tokens * per_tok + 2 * B * H * D * 2 + int((-(-ctx // 16)).sum()) * 4 + 4 * B

    shared = unique_bytes(W) < step_bytes(W)

    def launch_bytes(i):                       # the roofline's bytes of the attention pass
        return unique_bytes(i) if shared else step_bytes(i)

    def mean_bytes(steps, warmup, every=1):    # per launch over a run's timed steps
        return float(np.mean([launch_bytes(warmup + j) for j in range(0, steps, every)]))

    attn_bytes = float(np.mean([step_bytes(W + j) for j in sampled]))
    roof_bytes = mean_bytes(K, W, every)
    achieved = roof_bytes / (attn_avg_ms * 1e-3) / 1e9
    med, p10, p90 = (float(x) * 1e3 for x in np.percentile(attn_ms, [50, 10, 90]))
    log(f"{K} steps: wall {wall * 1e3:.2f} ms, events {gpu_ms:.2f} ms, attention pass "
        f"{attn_avg_ms * 1e3:.1f} us avg (median {med:.1f}, p10 {p10:.1f}, p90 {p90:.1f})")
    # the step decodes a batch of forked families as groups (one read of each shared block)
    kname = (f"decode_group_kernel<{wl.dtype_name.upper()},{D}" if batch.last_grouped
             else f"decode_attn_kernel<{wl.dtype_name.upper()},{D}") + (",FP8>" if fp8 else ">")
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof.update(traffic_fields(recorded_traffic(args) if bsz == 16 else None,
                               lambda s_, w_: mean_bytes(s_, w_)))
    roof.update({"kernel": kname, "avg_launch_us": round(attn_avg_ms * 1e3, 2),
                 "median_us": round(med, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2),
                 "samples": len(attn_ms), "bytes_per_launch": int(roof_bytes)})
    if flushed_ms:
        f_bytes = float(np.mean([launch_bytes(W + K + j) for j in range(F)]))
        f_avg = float(np.mean(flushed_ms))
        fm, f10, f90 = (float(x) * 1e3 for x in np.percentile(flushed_ms, [50, 10, 90]))
        roof["flushed_frac"] = round(f_bytes / (f_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        roof["flushed"] = {"avg_us": round(f_avg * 1e3, 2), "median_us": round(fm, 2),
                           "p10_us": round(f10, 2), "p90_us": round(f90, 2), "samples": F,
                           "bytes_per_launch": int(f_bytes),
                           "flush": f"{FLUSH_BYTES >> 20} MiB written before each launch"}
        log(f"flushed: {F} steps, attention pass {f_avg * 1e3:.1f} us avg (median {fm:.1f}, "
            f"p10 {f10:.1f}, p90 {f90:.1f}), frac {roof['flushed_frac']}")
    # the ceilings of the pass's own tiles (16-bit or FP8), where they are enough bytes to
    # time (not the tiny batch)
    if bsz == 16 and not args.no_ceiling and roof_bytes >= (64 << 20):
        roof["ceiling"] = read_ceiling(cache, sids, max_blocks, wl, dev, achieved)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype_name,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "num_heads": H, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": bsz, "kv_dtype": "fp8_e4m3" if fp8 else wl.dtype_name,
                   "context": CONTEXT_TEXT[wl.cfg_id],
                   "mean_context": round(float(base_ctx.mean() + W + (K - 1) / 2), 1),
                   "num_blocks": int(cache.num_blocks), "staging": batch.staging},
        "pool_waste": round(cache.bm.stats()["waste"], 4),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "seq_steps_per_s": round(B * K / wall, 1),
        "roofline": roof,
    }
    if shared:
        # aliased blocks: the roofline counts each shared block once (what HBM must
        # deliver); the logical rate counts it once per sequence that reads it
        result["roofline"]["accounting"] = "unique cached tokens (shared blocks once)"
        result["roofline"]["bytes_per_launch_logical"] = int(attn_bytes)
        result["roofline"]["achieved_logical"] = round(attn_bytes / (attn_avg_ms * 1e-3) / 1e9, 1)
    del cache, batch, steps_kv
    torch.cuda.empty_cache()
    if not args.no_other_ops:
        result["other_ops"] = other_ops(dev)
    if not args.no_cpu_baseline:
        log("CPU oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
