"""Build libgtf.so in-tree with hipcc for gfx950.

Host planning code (C++17) and the kernels (HIP) go into one shared
library next to this file.  Every HIP translation unit is compiled with
  -ffp-contract=off                          no multiply-add contraction, so
                                             chains of IEEE ops round like
                                             the op-by-op definition
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE division and square root
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                             no packed fp32 instructions
  -mllvm -simplifycfg-sink-common=false      keep the interpreter's per-slot
                                             cases apart: merging them turns
                                             constant register indices into
                                             pointer phis and forces the
                                             op-program stack into scratch
  -mllvm -structurizecfg-skip-uniform-regions=true
                                             leave the interpreter's dispatch
                                             switch (wave-uniform) a tree of
                                             scalar branches; structurised,
                                             every case writes a second copy
                                             of the register state
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgtf.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-ffp-contract=off",
          "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-simplifycfg-sink-common=false",
          "-mllvm", "-structurizecfg-skip-uniform-regions=true"]

SOURCES = ["plan.cpp", "bucket_plan.cpp", "capi.cpp", "kernels.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", *COMMON,
               "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"compile failed: {src}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
