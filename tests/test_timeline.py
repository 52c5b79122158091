"""The decode kernel's timeline (pa_timeline.h) on the host: the calls of the
ordinary build refuse, the instrumented build exports the same functions, and
the bench's summary of a launch's records reads hand-made records correctly."""

import ctypes as C
import glob
import os
import re

import numpy as np
import pytest

from tests.conftest import ROOT

N = pytest.importorskip("paged_kv_cache_385_amd._native")

TL_LIB = os.path.join(ROOT, "paged_kv_cache_385_amd", "libpa_timeline.so")


def _declared():
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text))
    return names


def test_ordinary_build_refuses_the_timeline_calls():
    lib = N.lib()
    buf = np.zeros((1, N.TIMELINE_WORDS), dtype=np.uint64)
    assert lib.pa_timeline_clear(None) == N.PA_ERR_UNSUPPORTED
    assert b"PA_TIMELINE" in lib.pa_last_error()
    assert lib.pa_timeline_read(buf.ctypes.data, 1) == N.PA_ERR_UNSUPPORTED
    assert lib.pa_timeline_read(buf.ctypes.data, 0) == N.PA_ERR_INVALID_ARG
    assert lib.pa_timeline_read(None, 1) == N.PA_ERR_INVALID_ARG
    assert lib.pa_timeline_read(buf.ctypes.data, N.TIMELINE_MAX_WORKGROUPS + 1) == N.PA_ERR_INVALID_ARG


@pytest.mark.skipif(not os.path.exists(TL_LIB), reason="libpa_timeline.so not built")
def test_instrumented_build_exports_every_declared_function():
    lib = C.CDLL(TL_LIB)
    for name in sorted(_declared()):
        assert hasattr(lib, name), name
    lib.pa_timeline_read.argtypes = [C.c_void_p, C.c_int32]
    buf = np.zeros((1, N.TIMELINE_WORDS), dtype=np.uint64)
    assert lib.pa_timeline_read(buf.ctypes.data, 0) == N.PA_ERR_INVALID_ARG


def _rec(entry, plan, first, loop, out, b, p, kg, nw0, tiles, xcc, cu, se=0):
    hw = (se << 13) | (cu << 8)
    return [entry, plan, first, loop, out, (b << 32) | p, (kg << 32) | (nw0 << 16) | tiles,
            (xcc << 32) | hw]


def test_timeline_summary_of_hand_made_records():
    import bench
    hz = bench.TIMELINE_HZ
    t = lambda us: int(1000 + us * hz / 1e6)                      # noqa: E731  (ticks)
    recs = np.zeros((8, N.TIMELINE_WORDS), dtype=np.uint64)
    # blockIdx 0: 0 -> 2 (plan) -> 7 (first tile) -> 47 (last) -> 50 (out); 9 tiles of wave 0
    recs[0] = _rec(t(0), t(2), t(7), t(47), t(50), 3, 0, 1, 9, 36, 0, 5)
    # blockIdx 1: starts at 10, 5 tiles of wave 0 (first at 20, last at 32: 3 us per tile)
    recs[1] = _rec(t(10), t(11), t(20), t(32), t(35), 4, 1, 0, 5, 20, 1, 5)
    # blockIdx 2 left unwritten; blockIdx 3: a wave 0 with no tile, on XCC 2 (3 mod 8 = 3)
    recs[3] = _rec(t(40), t(41), 0, t(41), t(60), 5, 0, 2, 0, 1, 2, 7)
    s = bench.timeline_summary(recs, event_us=61.0)
    assert s["workgroups"] == 3 and s["misordered"] == 0
    assert s["tiles_per_kv_head"] == 57
    assert s["span_us"] == pytest.approx(60.0)
    assert s["max_running"] == 2 and s["max_running_reached_us"] == pytest.approx(10.0)
    assert s["running_per_10us"] == [1, 2, 2, 2, 2, 1]
    assert s["plan_us"]["median"] == pytest.approx(1.0)
    # start-up of the two workgroups that streamed: 7 and 10 us
    assert s["startup_us"]["median"] == pytest.approx(8.5)
    assert s["first_tile_after_plan_us"]["median"] == pytest.approx(7.0)
    # pace of wave 0: (47 - 7) / 8 = 5 and (32 - 20) / 4 = 3
    assert s["wave0_us_per_tile"]["median"] == pytest.approx(4.0)
    assert s["per_xcc"] == [1, 1, 1, 0, 0, 0, 0, 0]
    assert s["xcc_of_block_mod_8"] == [[0], [1], [], [2], [], [], [], []]
    assert s["compute_units"] == 3
    # resident from the start (before the first output at 35 us): blocks 0 and 1, one per CU
    assert s["initial_per_cu"] == 1.0
    assert s["initial_startup_by_block_rank_us"] == [{"median": 8.5, "p90": 9.7}]
    # a record whose last tile precedes its first is counted as misordered
    recs[1, 3] = t(15)
    assert bench.timeline_summary(recs, 61.0)["misordered"] == 1
