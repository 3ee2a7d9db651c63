"""Build libssmscan.so: the HIP kernels and the C ABI, compiled by hipcc for gfx950.

Run as ``python -m mamba_selective_scan_s6_amd.build``.
The library is built in-tree, next to this file.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libssmscan.so")
# calibration kernels for bench.py's roofline denominators (not part of the scan library)
CAL_SRC = os.path.join(HERE, "calibrate", "rates.hip")
CAL_LIB = os.path.join(HERE, "libssmcal.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # packed FP32 instructions stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    # per-kernel register, scratch and occupancy figures, checked below
    "-Rpass-analysis=kernel-resource-usage",
]

# Occupancy floors the kernels are designed for, checked on every build, and every kernel runs without
# scratch. The scan kernel's latency hiding rests on 4 waves per SIMD (16 per CU); 3 for its
# zero-order-hold variants, whose gain needs 1/A per state in registers, and for the backward's
# checkpointing variants.
MIN_OCCUPANCY = {"scan_fwd_kernel": 4, "state_update_kernel": 4}
# mangled tails of scan instantiations with the zero-order-hold flag, or the checkpoint flag (the last
# two template flags) set: these may run at 3 waves per SIMD
OCC3_SCAN_SUFFIXES = ("Lb1ELb0EEEvNS0_6LbArgsE", "Lb0ELb1EEEvNS0_6LbArgsE")


def kernel_resources(stderr: str) -> dict:
    """Parse the compiler's kernel-resource-usage remarks into {kernel: {field: value}}."""
    out, cur = {}, None
    for line in stderr.splitlines():
        if "remark:" not in line or "kernel-resource-usage" not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[-Rpass-analysis", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = body.split(":", 1)[1].strip()
            out[cur] = {}
        elif cur is not None and ":" in body:
            k, v = body.rsplit(":", 1)
            out[cur][k.strip()] = v.strip()
    return out


def check_resources(res: dict) -> list:
    problems = []
    for name, r in res.items():
        for kern, occ in MIN_OCCUPANCY.items():
            if kern == "scan_fwd_kernel" and name.endswith(OCC3_SCAN_SUFFIXES):
                occ = 3
            if kern in name and int(r.get("Occupancy [waves/SIMD]", "0")) < occ:
                problems.append("%s: occupancy %s < %d (VGPRs %s)" % (name, r.get("Occupancy [waves/SIMD]"), occ,
                                                                      r.get("VGPRs")))
        if r.get("ScratchSize [bytes/lane]", "0") != "0" or r.get("VGPRs Spill", "0") != "0":
            problems.append("%s: uses scratch (%s bytes/lane, %s VGPRs spilled)" % (
                name, r.get("ScratchSize [bytes/lane]"), r.get("VGPRs Spill")))
    return problems


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


NOISE = ("unknown target feature", "packed-fp32-ops", "kernel-resource-usage")  # host pass / remarks


def _compile(hipcc: str, src: str, obj: str):
    cmd = [hipcc, *HIPCC_FLAGS, "-c", "-I", INCLUDE, "-I", CSRC, "-o", obj, src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    return cmd, res


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), check the kernels' resources, link."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda so: _compile(hipcc, *so), zip(srcs, objs)))
    stderr_all = ""
    for cmd, res in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        err = "\n".join(l for l in res.stderr.splitlines()
                        if not any(n in l for n in NOISE) and not l.lstrip().startswith(("|", "^"))
                        and not l.lstrip()[:1].isdigit())
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + err)
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        stderr_all += res.stderr + "\n"
    resources = kernel_resources(stderr_all)
    if not any("scan_fwd_kernel" in k for k in resources):
        raise RuntimeError("hipcc printed no kernel resource figures; cannot check the kernels")
    problems = check_resources(resources)
    if problems:
        raise RuntimeError("kernel resource check failed:\n  " + "\n  ".join(problems))
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs]
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("link failed:\n" + res.stderr)
    if verbose:
        print("%d kernels: %s" % (len(resources), ", ".join(sorted(
            {"VGPRs %s occ %s" % (r.get("VGPRs"), r.get("Occupancy [waves/SIMD]")) for r in resources.values()}))))
    os.replace(tmp, LIB)
    build_calibration(hipcc)
    return LIB


def build_calibration(hipcc: str) -> str:
    tmp = CAL_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-shared", "-o", tmp, CAL_SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed on the calibration kernels:\n" + res.stderr)
    os.replace(tmp, CAL_LIB)
    return CAL_LIB


if __name__ == "__main__":
    print(build(verbose=True))
