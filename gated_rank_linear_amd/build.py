"""Build libgsi.so (HIP, gfx950) in-tree: gated_rank_linear_amd/_lib/libgsi.so.

Run as `python -m gated_rank_linear_amd.build` or through __graft_entry__.build(). Every call
recompiles. Needs hipcc from ROCm; no GPU is needed to build.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libgsi.so")
BENCH_LIB = os.path.join(OUT_DIR, "libgsi_bench.so")
SOURCES = ["gsi_api.cpp", "gsi_dense.hip", "gsi_decode.hip", "gsi_calibrate.hip", "gsi_noalloc.hip", "gsi_step.hip"]

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # packed float32 VALU ops are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; ROCm is required to build libgsi")
    return p


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=gfx950", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libgsi failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    # the benchmark's streaming-read reference kernel, a library of its own (not libgsi's interface)
    tmp = BENCH_LIB + ".tmp"
    cmd = [cc, *HIP_FLAGS, "-x", "hip", "-shared", "-Wl,--no-undefined", os.path.join(CSRC, "bench_stream.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the stream-read kernel failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, BENCH_LIB)
    return LIB


PHASE_LIB = os.path.join(OUT_DIR, "libgsi_phases.so")


def build_phase_timeline() -> str:
    """A profiling variant of libgsi (_lib/libgsi_phases.so): the same sources with the batch-1
    kernel's phase stamps compiled in (GSI_PHASE_STAMPS) and gsi_phase_stamps exported. Used by
    gated_rank_linear_amd.phase_timeline only; libgsi itself never carries the stamps."""
    os.makedirs(OUT_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(OUT_DIR, "phases_" + os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIP_FLAGS, "-DGSI_PHASE_STAMPS", "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=gfx950", "-Wl,--no-undefined", *objs, "-o", PHASE_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    for o in objs:
        os.remove(o)
    if r.returncode != 0:
        raise RuntimeError(f"linking the phase-stamp library failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return PHASE_LIB


if __name__ == "__main__":
    if "--phase-stamps" in sys.argv[1:]:
        print(build_phase_timeline())
    else:
        print(build(verbose=True))
