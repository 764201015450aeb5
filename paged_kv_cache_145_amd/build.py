"""Build the gfx950 shared library ``libpa_mi355x.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled, then linked with the plain C++ allocator into one shared
object next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libpa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# Measurement build: the same library with per-wave timeline stamps in the
# stream-K decode kernels (PA_WAVE_TIMELINE); only `bench.py --timeline`
# loads it.
TIMELINE_LIB_NAME = "libpa_mi355x_timeline.so"
TIMELINE_LIB_PATH = os.path.join(PKG, TIMELINE_LIB_NAME)
TIMELINE_SOURCES = ["decode_kernels.hip", "multi_kernels.hip", "api.hip"]  # the files the define changes

HIP_SOURCES = ["decode_kernels.hip", "multi_kernels.hip", "write_kernels.hip", "api.hip"]
CPP_SOURCES = ["pool.cpp", "prefix.cpp", "batching.cpp"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    # MFMA accumulators in ordinary VGPRs: with the accumulation registers
    # (AGPRs) the compiler copied the multi-token kernel's 96 output
    # accumulators out and back on every key tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    return proc


def _link(hipcc, objs, path, verbose):
    tmp = path + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, path)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link ``libpa_mi355x.so`` and the timeline
    measurement library; returns the product library's path."""
    hipcc = _hipcc()
    tl_dir = os.path.join(BUILD_DIR, "timeline")
    os.makedirs(tl_dir, exist_ok=True)
    cmds = []
    objs = []
    tl_objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmds.append([hipcc, *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
        if src in TIMELINE_SOURCES:
            tl_obj = os.path.join(tl_dir, src + ".o")
            cmds.append([hipcc, *COMMON, *HIP_FLAGS, "-DPA_WAVE_TIMELINE", "-c", os.path.join(CSRC, src),
                         "-o", tl_obj])
            tl_objs.append(tl_obj)
        else:
            tl_objs.append(obj)
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmds.append([hipcc, *COMMON, "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
        tl_objs.append(obj)
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _link(hipcc, objs, LIB_PATH, verbose)
    _link(hipcc, tl_objs, TIMELINE_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
