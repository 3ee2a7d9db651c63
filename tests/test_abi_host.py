"""The C-ABI library on the host: it loads, exports every function include/*.h declares, and
rejects invalid arguments with the documented status before any HIP call (no GPU needed: no
valid compute call is made here)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from conftest import ROOT

LIB = os.path.join(ROOT, "mamba_selective_scan_s6_amd", "libssmscan.so")
SSM_OK, NULLP, SHAPE, DTYPE, ALIGN, HIP, WAIT, FLAGS = 0, 1, 2, 3, 4, 5, 6, 7
FLAG_ZOH = 1


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \t\*]*?\b(ssm_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libssmscan.so is not built (python -m mamba_selective_scan_s6_amd.build)")
    import mamba_selective_scan_s6_amd as m

    return m.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ssm_scan_fwd", "ssm_state_update", "ssm_status_string", "ssm_last_error_message", "ssm_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in declared_functions():
        assert n in exported, "%s declared in include/ but not exported" % n
        assert hasattr(lib, n)


def test_segment_length(lib):
    """Workgroups take 64-token segments of 64 channels whatever the shape; invalid sizes give 0.
    No HIP call is made."""
    for shape in ((1, 64, 128), (1, 1536, 2048), (4, 5120, 2048), (1, 2048, 65536), (3, 7, 5)):
        assert lib.ssm_scan_segment_tokens(*shape) == 64
    assert lib.ssm_scan_segment_tokens(0, 64, 128) == 0
    assert lib.ssm_scan_segment_tokens(1, 64, 0) == 0


def test_version_and_status_strings(lib):
    assert lib.ssm_abi_version() == 2
    assert lib.ssm_status_string(ALIGN) == b"SSM_ERR_MISALIGNED"
    assert lib.ssm_status_string(FLAGS) == b"SSM_ERR_BAD_FLAGS"
    assert lib.ssm_status_string(99) == b"SSM_ERR_UNKNOWN"


# Fake, never-dereferenced device addresses: validation only looks at their values.
P = 0x7F0000000000
OK_ARGS = dict(u=P, delta=P + 0x100000, A=P + 0x200000, B=P + 0x300000, C=P + 0x400000, D=None, z=None,
               delta_bias=None, softplus=1, out=P + 0x500000, last_state=None, nb=1, nd=64, L=128, N=16, io=0)


def scan(lib, **kw):
    a = dict(OK_ARGS)
    a.update(kw)
    return lib.ssm_scan_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["delta_bias"], a["softplus"],
                            a["out"], a["last_state"], a["nb"], a["nd"], a["L"], a["N"], a["io"], None)


@pytest.mark.parametrize("field", ["u", "delta", "A", "B", "C", "out"])
def test_scan_rejects_null(lib, field):
    assert scan(lib, **{field: None}) == NULLP
    assert field in lib.ssm_last_error_message().decode()


@pytest.mark.parametrize("kw", [dict(nb=0), dict(nd=0), dict(L=0), dict(N=0), dict(N=17), dict(nb=-3),
                                dict(nb=1 << 40, nd=1 << 40)])
def test_scan_rejects_bad_shape(lib, kw):
    assert scan(lib, **kw) == SHAPE


def test_scan_rejects_bad_dtype(lib):
    assert scan(lib, io=2) == DTYPE
    assert scan(lib, io=-1) == DTYPE


@pytest.mark.parametrize("field", ["u", "delta", "A", "B", "C", "D", "z", "delta_bias", "out", "last_state"])
def test_scan_rejects_misaligned(lib, field):
    base = OK_ARGS[field] or (P + 0x900000)
    assert scan(lib, **{field: base + 4}) == ALIGN


def test_scan_rejects_aliasing_output(lib):
    assert scan(lib, out=OK_ARGS["u"]) == SHAPE
    assert scan(lib, out=OK_ARGS["delta"] + 64) == SHAPE


def test_error_message_is_thread_local_detail(lib):
    assert scan(lib, N=99) == SHAPE
    assert b"dstate=99" in lib.ssm_last_error_message()


def update(lib, **kw):
    a = dict(state=P, x=P + 0x100000, delta=P + 0x200000, A=P + 0x300000, B=P + 0x400000, C=P + 0x500000, D=None,
             z=None, out=P + 0x600000, nb=2, nd=64, N=16, io=1)
    a.update(kw)
    return lib.ssm_state_update(a["state"], a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["out"],
                                a["nb"], a["nd"], a["N"], a["io"], None)


def scan_ex(lib, flags, **kw):
    a = dict(OK_ARGS)
    a.update(kw)
    return lib.ssm_scan_fwd_ex(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["delta_bias"],
                               a["softplus"], a["out"], a["last_state"], a["nb"], a["nd"], a["L"], a["N"], a["io"],
                               flags, None)


def update_ex(lib, flags, **kw):
    a = dict(state=P, x=P + 0x100000, delta=P + 0x200000, A=P + 0x300000, B=P + 0x400000, C=P + 0x500000, D=None,
             z=None, out=P + 0x600000, nb=2, nd=64, N=16, io=1)
    a.update(kw)
    return lib.ssm_state_update_ex(a["state"], a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["out"],
                                   a["nb"], a["nd"], a["N"], a["io"], flags, None)


@pytest.mark.parametrize("flags", [2, 4, 0x80000000, FLAG_ZOH | 2])
def test_ex_entry_points_reject_unknown_flags(lib, flags):
    assert scan_ex(lib, flags) == FLAGS
    assert b"flag" in lib.ssm_last_error_message()
    assert update_ex(lib, flags) == FLAGS


def test_ex_entry_points_validate_like_the_plain_ones(lib):
    # the flag is accepted; the other checks still apply before any HIP call
    assert scan_ex(lib, FLAG_ZOH, N=0) == SHAPE
    assert scan_ex(lib, FLAG_ZOH, u=None) == NULLP
    assert update_ex(lib, FLAG_ZOH, io=7) == DTYPE
    assert update_ex(lib, 0, z=P + 0x700002) == ALIGN


@pytest.mark.parametrize("field", ["state", "x", "delta", "A", "B", "C", "out"])
def test_update_rejects_null(lib, field):
    assert update(lib, **{field: None}) == NULLP


def test_update_rejects_shape_dtype_alignment(lib):
    assert update(lib, nb=0) == SHAPE
    assert update(lib, N=17) == SHAPE
    assert update(lib, io=5) == DTYPE
    assert update(lib, z=P + 0x700002) == ALIGN
    assert update(lib, out=P) == SHAPE  # out inside state


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import importlib

    import mamba_selective_scan_s6_amd as m

    monkeypatch.setattr(m, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(m, "_lib", None)
    with pytest.raises(ImportError):
        m.load_library()
    importlib.reload(m)


def conv(lib, **kw):
    a = dict(x=P, w=P + 0x100000, b=None, silu=1, out=P + 0x200000, nb=2, nd=64, L=100, K=4, io=0)
    a.update(kw)
    return lib.ssm_causal_conv1d(a["x"], a["w"], a["b"], a["silu"], a["out"], a["nb"], a["nd"], a["L"], a["K"], a["io"],
                                 None)


def window(lib, **kw):
    a = dict(win=P, x=P + 0x100000, w=P + 0x200000, b=None, silu=1, out=P + 0x300000, nb=2, nd=64, K=4, io=1)
    a.update(kw)
    return lib.ssm_conv_window_update(a["win"], a["x"], a["w"], a["b"], a["silu"], a["out"], a["nb"], a["nd"], a["K"],
                                      a["io"], None)


def test_conv_entry_points_validate(lib):
    for f in ("x", "w", "out"):
        assert conv(lib, **{f: None}) == NULLP
    for kw in (dict(K=0), dict(K=9), dict(L=0), dict(nb=0), dict(nb=1 << 40, nd=1 << 40)):
        assert conv(lib, **kw) == SHAPE
    assert conv(lib, io=3) == DTYPE
    assert conv(lib, b=P + 0x300008) == ALIGN
    assert conv(lib, out=P + 64) == SHAPE  # out inside x
    for f in ("win", "x", "w", "out"):
        assert window(lib, **{f: None}) == NULLP
    assert window(lib, K=9) == SHAPE
    assert window(lib, io=-1) == DTYPE
    assert window(lib, out=P) == SHAPE  # out inside the window
    assert b"width" in (conv(lib, K=12) == SHAPE and lib.ssm_last_error_message())


def test_wait_limit_knob(lib):
    """The look-back's poll limit can be set and restored; <= 0 selects the default. No HIP call."""
    default = lib.ssm_set_wait_limit(7)
    assert default > 1000
    assert lib.ssm_set_wait_limit(0) == 7
    assert lib.ssm_set_wait_limit(-3) == default
    assert lib.ssm_set_wait_limit(0) == default


def bwd(lib, **kw):
    a = dict(u=P, delta=P + 0x100000, A=P + 0x200000, B=P + 0x300000, C=P + 0x400000, D=None, z=None, bias=None,
             sp=1, dout=P + 0x500000, du=P + 0x600000, ddelta=P + 0x700000, dA=P + 0x800000, dB=P + 0x900000,
             dC=P + 0xA00000, dD=None, dz=None, dbias=None, nb=1, nd=64, L=128, N=16, io=0)
    a.update(kw)
    return lib.ssm_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"], a["dout"],
                            a["du"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"], a["dbias"], a["nb"],
                            a["nd"], a["L"], a["N"], a["io"], None)


def test_scan_bwd_validates(lib):
    for f in ("u", "delta", "A", "B", "C", "dout", "du", "ddelta", "dA", "dB", "dC"):
        assert bwd(lib, **{f: None}) == NULLP, f
    assert bwd(lib, z=P + 0xB00000) == NULLP  # dz is required with z
    assert b"dz" in lib.ssm_last_error_message()
    for kw in (dict(N=0), dict(N=17), dict(L=0), dict(nb=1 << 40, nd=1 << 40)):
        assert bwd(lib, **kw) == SHAPE
    assert bwd(lib, io=9) == DTYPE
    assert bwd(lib, dA=P + 0x800004) == ALIGN
    assert bwd(lib, du=P + 0x100000) == SHAPE  # du overlaps delta
