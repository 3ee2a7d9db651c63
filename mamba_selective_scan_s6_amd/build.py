"""Build libssmscan.so: the HIP kernels and the C ABI, compiled by hipcc for gfx950.

Run as ``python -m mamba_selective_scan_s6_amd.build`` (or through ``__graft_entry__.build()``).
The library is built in-tree, next to this file.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssmscan.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
    # packed FP32 instructions stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "unknown target feature"  # the host pass does not know the device-only feature
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
