"""The decode kernel's per-workgroup timeline (libpa_timeline.so, pa_timeline.h) on
the 70B-shaped GQA-8 decode layer: the bench's capture runs in a child process
(the instrumented library replaces libpa.so there), and each captured launch's
records must account for every context tile exactly once, be ordered in time
and fit inside the events around the launch."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

from tests.conftest import ROOT

pytestmark = pytest.mark.gpu

TL_LIB = os.path.join(ROOT, "paged_kv_cache_385_amd", "libpa_timeline.so")


def test_timeline_accounts_for_every_tile(tmp_path):
    import bench
    from workloads import make_workload
    assert os.path.exists(TL_LIB), "libpa_timeline.so is not built"
    steps, warmup = 2, 1
    out = tmp_path / "timeline.json"
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "3",
           "--steps", str(steps), "--warmup", str(warmup), "--flush-steps", "0",
           "--no-cpu-baseline", "--no-other-ops", "--no-ceiling", "--timeline", str(out)]
    print("child:", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    d = json.load(open(out))
    assert d["library"] == "libpa_timeline.so"
    wl = make_workload(3, grow=steps + warmup + bench.TIMELINE_STEPS)
    assert len(d["launches"]) == bench.TIMELINE_STEPS
    for t in d["launches"]:
        print({k: t[k] for k in ("step", "workgroups", "span_us", "event_us", "max_running",
                                 "compute_units", "xcc_of_block_mod_8")}, flush=True)
        ctx = wl.ctx_lens.astype(np.int64) + t["step"]
        # one item per (sequence, KV head, partition); its tiles are that partition's blocks
        assert t["tiles_per_kv_head"] == wl.num_kv_heads * int((-(-ctx // 16)).sum())
        assert t["misordered"] == 0
        # the stamps' clock: the pass fits inside the launch's events and fills most of it
        assert 0.7 * t["event_us"] <= t["span_us"] <= t["event_us"] + 2.0
        assert sum(t["per_xcc"]) == t["workgroups"]
        # blocks are dealt to the XCDs in turn: each residue mod 8 runs on one XCC
        assert all(len(x) == 1 for x in t["xcc_of_block_mod_8"]), t["xcc_of_block_mod_8"]
