"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two executables are built from source with gcc/g++ and run:
  * the C ABI's argument checks (csrc/abi.cpp, instrumented) driven through every rejection path and
    the size queries, linked against the built library for the kernels' host-side size helpers (no
    HIP call is reached: every call is invalid or a pure query);
  * the fp64 oracle (oracle/oracle.c, instrumented) on ragged shapes with exact-size allocations.
Any sanitizer report makes the run exit non-zero."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
CSRC = os.path.join(ROOT, "mamba_selective_scan_s6_amd", "csrc")
LIBDIR = os.path.join(ROOT, "mamba_selective_scan_s6_amd")
HERE = os.path.join(ROOT, "tests", "sanitize")


def _compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip("%s is not installed" % name)
    return path


def _run(exe, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    return res.stdout


def test_abi_validation_under_sanitizers(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libssmscan.so")):
        pytest.fail("libssmscan.so is not built (python -m mamba_selective_scan_s6_amd.build)")
    gxx = _compiler("g++")
    gcc = _compiler("gcc")
    obj = str(tmp_path / "driver.o")
    exe = str(tmp_path / "abi_validation")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    subprocess.run([gcc, *SAN, *inc, "-c", "-o", obj, os.path.join(HERE, "abi_validation.c")], check=True)
    subprocess.run([gxx, *SAN, "-std=c++17", *inc, "-o", exe, os.path.join(CSRC, "abi.cpp"), obj,
                    "-L", LIBDIR, "-lssmscan", "-Wl,-rpath," + LIBDIR, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-lpthread"], check=True)
    # leak checking stays off here: the HIP runtime's own start-up allocations are not this code's
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert "abi validation ok" in out


def test_oracle_under_sanitizers(tmp_path):
    gcc = _compiler("gcc")
    exe = str(tmp_path / "oracle_memcheck")
    subprocess.run([gcc, *SAN, "-std=c11", "-ffp-contract=off", "-o", exe, os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(HERE, "oracle_memcheck.c"), "-lm", "-lpthread"], check=True)
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=1", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert "oracle memcheck ok" in out
