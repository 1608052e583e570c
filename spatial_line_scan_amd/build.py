"""Build libgspn.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

    python -m spatial_line_scan_amd.build

Every HIP translation unit is compiled for gfx950 only, with packed-fp32
instruction selection turned off (plain fp32 VALU ops).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgspn.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["gspn_host.cpp", "gspn_kernels.hip", "gspn_prop2d_pair.hip", "gspn_prop2d_phase.hip", "gspn_prop2d_quad.hip", "gspn_prop2d_duo.hip",
           "gspn_backward.hip", "gspn_backward_pair.hip", "gspn_sublayer.hip", "gspn_conv1x1.hip",
           "gspn_prop2d_wide.hip", "gspn_backward_wide.hip", "gspn_noalloc.hip",
           "gspn_scan_dir.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _jobs() -> int:
    """Parallel compiles: MAX_JOBS if set, else the CPUs this process may use."""
    env = os.environ.get("MAX_JOBS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return os.cpu_count() or 1


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libgspn.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(_jobs(), len(cmds))) as pool:
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
        # check_call raises on the first failed compile, after the others end
        list(pool.map(subprocess.check_call, cmds))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp,
           "-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
