"""Builds libzc.so (HIP, gfx950) in-tree.

Steps:
  1. compile and run the table emitter (host C++), which computes the code
     table of table_id 1 from the closed-form law and writes its constants;
  2. compile the kernels and the C ABI with hipcc for gfx950.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libzc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # keep packed fp32 instructions out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # a single-lane atomic stays one atomic whose result is waited for where
    # it is used (the optimizer's wave reduction waits at once)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: %s" % " ".join(cmd[:3]))
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    emit = os.path.join(BUILD, "zc_table_emit")
    _run(["g++", "-O2", "-std=c++17", "-Wall", "-o", emit,
          os.path.join(CSRC, "zc_table.cpp"), os.path.join(CSRC, "zc_table_emit.cpp")])
    inc = _run([emit])
    with open(os.path.join(BUILD, "zc_table_v1.inc"), "w") as f:
        f.write(inc)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *HIP_FLAGS, "-shared",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", BUILD,
           os.path.join(CSRC, "zc_kernels.hip"), os.path.join(CSRC, "zc_table.cpp"),
           os.path.join(CSRC, "zc_switch.cpp"),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
