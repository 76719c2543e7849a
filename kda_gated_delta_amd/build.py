"""Builds libkda.so (all HIP sources under csrc/) and libkda_probe.so (the
measured-ceiling kernels under probe/) for gfx950, in-tree.

hipcc compiles every translation unit for gfx950 only, with packed-fp32
instructions disabled, and links them into one shared library next to this
file.  Run as ``python -m kda_gated_delta_amd.build`` or via
``__graft_entry__.build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkda.so")
PROBE_DIR = os.path.join(HERE, "probe")
PROBE_LIB = os.path.join(HERE, "libkda_probe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = ["hipcc", *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 4) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe_srcs = sorted(glob.glob(os.path.join(PROBE_DIR, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs + probe_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 4))
