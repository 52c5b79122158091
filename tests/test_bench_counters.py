"""bench.py's HBM-counter summary on synthetic rocprofv3 counter files (no GPU).

The summary scales each counter by what it read for a calibration copy of known size,
takes the timed calls (after the warm-up calls, before the flushed ones; a call may be an
attention and a merge launch), and stamps
the result with the kernel source; the bench line uses it only while the stamp and the workload
match, and reports it with the counter run's own algorithmic bytes.
"""

import csv
import json
import types

import bench


def _counter_csv(path, name, calib_value, launches, values):
    """3 calibration copies, then the launches (kernel name, value) in dispatch order."""
    rows = []
    did = 1
    for _ in range(3):
        rows.append(dict(Dispatch_Id=did, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name=name,
                         Counter_Value=calib_value))
        did += 1
    for k, v in zip(launches, values):
        rows.append(dict(Dispatch_Id=did, Kernel_Name=k, Counter_Name=name, Counter_Value=v))
        did += 1
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _args(tmp_path, chunk, fetch, write, steps=4, warmup=2, flush_steps=0):
    return types.SimpleNamespace(chunk=chunk, workload=3, steps=steps, warmup=warmup,
                                 flush_steps=flush_steps, kv_dtype="native", copy_calibration=1,
                                 summarize_counters=[str(fetch), str(write)])


def _leg(chunk=None, workload=3, kv_dtype="native"):
    return types.SimpleNamespace(chunk=chunk, workload=workload, kv_dtype=kv_dtype)


def test_decode_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    out = tmp_path / "decode_{mode}.json"
    path, src, names = bench.TRAFFIC["decode"]
    monkeypatch.setitem(bench.TRAFFIC, "decode", (str(out), src, names))
    k = "void decode_attn_kernel<BF16, 128>(DecodeArgs)"
    # a 1 MiB copy reads as 512 KiB of FETCH_SIZE (scale 2) and 1024 KiB of WRITE_SIZE
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", 512, [k] * 6, [9, 9, 100, 100, 110, 110])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", 1024, [k] * 6, [1, 1, 4, 4, 4, 4])
    bench.summarize_counters(_args(tmp_path, None, tmp_path / "f.csv", tmp_path / "w.csv"))
    t = json.loads((tmp_path / "decode_w3.json").read_text())
    assert t["workload"] == "w3"
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["launches"] == 4                                 # the warm-up launches are dropped
    assert t["fetch_bytes_per_launch"] == int(105 * 1024 * 2)
    assert t["write_bytes_per_launch"] == 4 * 1024
    assert t["traffic_bytes_per_launch"] == 105 * 2048 + 4096
    assert t["source_sha256"] == bench.source_sha256(src)
    rec = bench.recorded_traffic(_leg())
    assert rec["traffic_bytes_per_launch"] == t["traffic_bytes_per_launch"]
    assert bench.recorded_traffic(_leg(workload=2)) is None            # another workload
    assert bench.recorded_traffic(_leg(kv_dtype="fp8")) is None        # another pool type
    # the bench line: the counter run's bytes, and their ratio to that run's algorithmic bytes
    seen = []

    def alg(steps, warmup):
        seen.append((steps, warmup))
        return 105 * 1024
    f = bench.traffic_fields(rec, alg)
    assert seen == [(4, 2)]
    assert f["traffic"] == t["traffic_bytes_per_launch"]
    assert f["traffic_ratio"] == round((105 * 2048 + 4096) / (105 * 1024), 4)
    assert bench.traffic_fields(None, alg) == {"traffic": None}


def test_chunk_summary_sums_the_launches_of_a_call(tmp_path, monkeypatch):
    out = tmp_path / "chunk_{mode}.json"
    path, src, names = bench.TRAFFIC["chunk"]
    monkeypatch.setitem(bench.TRAFFIC, "chunk", (str(out), src, names))
    a, m = "chunk_attn_kernel<BF16, 128, 3, true, false>", "chunk_merge_kernel<BF16, 128>"
    calls = [a, m] * 6                                        # 2 warm-up + 4 timed calls
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", 512, calls, [50, 5] * 6)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", 1024, calls, [3, 1] * 6)
    bench.summarize_counters(_args(tmp_path, "verify", tmp_path / "f.csv", tmp_path / "w.csv"))
    t = json.loads((tmp_path / "chunk_verify.json").read_text())
    assert t["workload"] == "chunk-verify" and t["launches"] == 8
    assert t["fetch_bytes_per_launch"] == 55 * 1024 * 2       # per call: attention + merge
    assert t["write_bytes_per_launch"] == 4 * 1024
    assert bench.recorded_traffic(_leg("verify"))["traffic_bytes_per_launch"] \
        == t["traffic_bytes_per_launch"]
    assert bench.recorded_traffic(_leg("prefill")) is None


def test_decode_summary_drops_the_flushed_steps(tmp_path, monkeypatch):
    import pytest
    out = tmp_path / "decode_{mode}.json"
    path, src, names = bench.TRAFFIC["decode"]
    monkeypatch.setitem(bench.TRAFFIC, "decode", (str(out), src, names))
    k = "void decode_group_kernel<F16, 128, true, false>(GroupArgs)"
    # 2 warm-up, 4 timed and 3 flushed steps: only the timed ones count
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", 1024, [k] * 9, [1, 1, 10, 10, 10, 10, 99, 99, 99])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", 1024, [k] * 9, [2] * 9)
    bench.summarize_counters(_args(tmp_path, None, tmp_path / "f.csv", tmp_path / "w.csv",
                                   flush_steps=3))
    t = json.loads((tmp_path / "decode_w3.json").read_text())
    assert t["launches"] == 4 and t["fetch_bytes_per_launch"] == 10 * 1024
    with pytest.raises(SystemExit):            # the counter runs had other --flush-steps
        bench.summarize_counters(_args(tmp_path, None, tmp_path / "f.csv", tmp_path / "w.csv"))
