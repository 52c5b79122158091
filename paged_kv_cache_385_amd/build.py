"""Build libpa.so in-tree: HIP kernels for gfx950 plus the host block manager.
Also builds libpa_timeline.so, the same library whose decode kernel records a
per-workgroup timeline (pa_timeline.h).

    python -m paged_kv_cache_385_amd.build

Every call compiles from source (no staleness check).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
# the same library with the decode kernel's per-workgroup timeline (pa_timeline.h)
LIB_TIMELINE = os.path.join(PKG, "libpa_timeline.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ops disabled in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, save_temps: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    bm_o = os.path.join(BUILD, "block_manager.o")
    k_o = os.path.join(BUILD, "pa_kernels.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", *inc, "-c",
          os.path.join(CSRC, "block_manager.cpp"), "-o", bm_o], verbose)
    step_o = os.path.join(BUILD, "decode_step.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__", *inc,
          "-I", "/opt/rocm/include", "-c", os.path.join(CSRC, "decode_step.cpp"), "-o", step_o],
         verbose)
    extra = ["-save-temps=obj"] if save_temps else []
    _run([hipcc, *HIP_FLAGS, *inc, *extra, "-c", os.path.join(CSRC, "pa_kernels.hip"), "-o", k_o],
         verbose)
    c_o = os.path.join(BUILD, "chunk_attention.o")
    _run([hipcc, *HIP_FLAGS, *inc, *extra, "-c", os.path.join(CSRC, "chunk_attention.hip"), "-o",
          c_o], verbose)
    n_o = os.path.join(BUILD, "decode_noalloc.o")
    _run([hipcc, *HIP_FLAGS, *inc, *extra, "-c", os.path.join(CSRC, "decode_noalloc.hip"), "-o",
          n_o], verbose)
    gp_o = os.path.join(BUILD, "group_plan.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", *inc, "-c",
          os.path.join(CSRC, "group_plan.cpp"), "-o", gp_o], verbose)
    g_o = os.path.join(BUILD, "decode_grouped.o")
    _run([hipcc, *HIP_FLAGS, *inc, *extra, "-c", os.path.join(CSRC, "decode_grouped.hip"), "-o",
          g_o], verbose)
    p_o = os.path.join(BUILD, "hbm_probe.o")
    _run([hipcc, *HIP_FLAGS, *inc, *extra, "-c", os.path.join(CSRC, "hbm_probe.hip"), "-o", p_o],
         verbose)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", bm_o, step_o, k_o, c_o, n_o, p_o,
          gp_o, g_o, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    tl_o = os.path.join(BUILD, "pa_kernels_timeline.o")
    _run([hipcc, *HIP_FLAGS, *inc, "-DPA_TIMELINE", "-c", os.path.join(CSRC, "pa_kernels.hip"),
          "-o", tl_o], verbose)
    tmp = LIB_TIMELINE + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", bm_o, step_o, tl_o, c_o, n_o, p_o,
          gp_o, g_o, "-o", tmp], verbose)
    os.replace(tmp, LIB_TIMELINE)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, save_temps="--save-temps" in sys.argv))
