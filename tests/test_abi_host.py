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
SSM_OK, NULLP, SHAPE, DTYPE, ALIGN, HIP, WAIT, FLAGS, WSP = 0, 1, 2, 3, 4, 5, 6, 7, 8
FLAG_ZOH, FLAG_OUT_F32 = 1, 2


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
    assert lib.ssm_abi_version() == 4
    assert lib.ssm_status_string(ALIGN) == b"SSM_ERR_MISALIGNED"
    assert lib.ssm_status_string(FLAGS) == b"SSM_ERR_BAD_FLAGS"
    assert lib.ssm_status_string(WSP) == b"SSM_ERR_WORKSPACE"
    assert lib.ssm_status_string(99) == b"SSM_ERR_UNKNOWN"


# Fake, never-dereferenced device addresses: validation only looks at their values.
P = 0x7F0000000000
WS = P + 0x10000000  # a fake workspace far from the tensors
OK_ARGS = dict(u=P, delta=P + 0x100000, A=P + 0x200000, B=P + 0x300000, C=P + 0x400000, D=None, z=None,
               delta_bias=None, softplus=1, out=P + 0x500000, last_state=None, nb=1, nd=64, L=128, N=16, io=0,
               ws=WS, ws_bytes=1 << 20)


def scan(lib, **kw):
    a = dict(OK_ARGS)
    a.update(kw)
    return lib.ssm_scan_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["delta_bias"], a["softplus"],
                            a["out"], a["last_state"], a["nb"], a["nd"], a["L"], a["N"], a["io"], a["ws"], a["ws_bytes"],
                            None)


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
                               flags, a["ws"], a["ws_bytes"], None)


def update_ex(lib, flags, **kw):
    a = dict(state=P, x=P + 0x100000, delta=P + 0x200000, A=P + 0x300000, B=P + 0x400000, C=P + 0x500000, D=None,
             z=None, out=P + 0x600000, nb=2, nd=64, N=16, io=1)
    a.update(kw)
    return lib.ssm_state_update_ex(a["state"], a["x"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["out"],
                                   a["nb"], a["nd"], a["N"], a["io"], flags, None)


@pytest.mark.parametrize("flags", [4, 8, 0x80000000, FLAG_ZOH | 4, FLAG_OUT_F32 | 16])
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
             dC=P + 0xA00000, dD=None, dz=None, dbias=None, nb=1, nd=64, L=128, N=16, io=0, ws=WS, ws_bytes=1 << 24)
    a.update(kw)
    return lib.ssm_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["sp"], a["dout"],
                            a["du"], a["ddelta"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"], a["dbias"], a["nb"],
                            a["nd"], a["L"], a["N"], a["io"], a["ws"], a["ws_bytes"], None)


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
    assert bwd(lib, ws=None) == WSP
    assert bwd(lib, ws_bytes=lib.ssm_scan_bwd_workspace_size(1, 64, 128) - 1) == WSP
    assert bwd(lib, ws=P + 0x800000) == WSP  # the workspace would cover dA


def test_workspace_size_query(lib):
    """The forward's workspace: a 256-byte header, then one 8704-byte slot (a flag row, the aggregate's
    17 rows and the inclusive state's 16 rows of 64 fp32 channels) per 64-token segment of every
    64-channel group of every batch row. Invalid sizes give 0. No HIP call is made."""
    slot = 256 * (1 + 17 + 16)
    for (nb, nd, L) in ((1, 64, 128), (1, 1536, 2048), (4, 5120, 2048), (1, 2048, 65536), (3, 7, 5), (2, 65, 65)):
        segs = nb * ((nd + 63) // 64) * ((L + 63) // 64)
        assert lib.ssm_scan_fwd_workspace_size(nb, nd, L) == 256 + segs * slot
        assert lib.ssm_scan_bwd_workspace_size(nb, nd, L) > lib.ssm_scan_fwd_workspace_size(nb, nd, L)
    for bad in ((0, 64, 128), (1, 0, 128), (1, 64, 0), (-1, 64, 128), (1 << 40, 1 << 40, 1)):
        assert lib.ssm_scan_fwd_workspace_size(*bad) == 0
        assert lib.ssm_scan_bwd_workspace_size(*bad) == 0


def test_scan_rejects_bad_workspace(lib):
    need = lib.ssm_scan_fwd_workspace_size(1, 64, 128)
    assert scan(lib, ws=None) == WSP
    assert b"NULL" in lib.ssm_last_error_message()
    assert scan(lib, ws_bytes=need - 1) == WSP
    assert b"needs" in lib.ssm_last_error_message()
    assert scan(lib, ws=WS + 8) == ALIGN
    assert scan(lib, ws=P + 0x500000 - 1024, ws_bytes=need) == WSP  # would run into out
    assert b"overlaps" in lib.ssm_last_error_message()
    assert scan_ex(lib, FLAG_ZOH, ws=None) == WSP
    # valid sizes pass every check that needs no GPU (the launch itself is not reached here)
    assert lib.ssm_scan_fwd_workspace_size(1, 64, 128) == need


def test_out_f32_flag_changes_the_output_extent(lib):
    """With SSM_FLAG_OUT_F32 a bf16 scan's out holds 4-byte elements. An out that ends exactly where
    delta starts when it holds bf16 passes the overlap checks (and is then refused only for the missing
    workspace); as fp32 it runs into delta."""
    elems = 1 * 64 * 128
    a = dict(io=1, u=P, delta=P + 0x100000, out=P + 0x100000 - elems * 2, ws=None)
    assert scan_ex(lib, 0, **a) == WSP
    assert scan_ex(lib, FLAG_OUT_F32, **a) == SHAPE
    assert b"out overlaps" in lib.ssm_last_error_message()


def test_noalloc_entry_point_refuses_problems_beyond_its_array(lib):
    """ssm_scan_fwd_noalloc validates like ssm_scan_fwd, then refuses a problem whose workspace exceeds
    its 64 MiB device array (here the long-context shape, 32 groups x 1024 segments), before any HIP
    call."""
    import ctypes

    vp, i64, ci, cu = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint
    lib.ssm_scan_fwd_noalloc.restype = ci
    lib.ssm_scan_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, vp, vp, i64, i64, i64, i64, ci, cu, vp]
    lib.ssm_scan_fwd_noalloc_max_workspace.restype = ctypes.c_size_t
    assert lib.ssm_scan_fwd_noalloc_max_workspace() == 64 << 20
    G = 1 << 30  # tensors 1 GiB apart: no overlap for these sizes
    args = [P, P + G, P + 2 * G, P + 3 * G, P + 4 * G, None, None, None, 1, P + 5 * G, None]
    assert lib.ssm_scan_fwd_noalloc(*args, 1, 2048, 65536, 16, 1, 0, None) == WSP
    assert b"ssm_scan_fwd_noalloc" in lib.ssm_last_error_message()
    assert lib.ssm_scan_fwd_workspace_size(1, 2048, 65536) > (64 << 20)
    # the other checks come first
    assert lib.ssm_scan_fwd_noalloc(*args, 1, 2048, 65536, 17, 1, 0, None) == SHAPE
    assert lib.ssm_scan_fwd_noalloc(*args, 1, 2048, 65536, 16, 1, 4, None) == FLAGS


def test_every_written_tensor_is_checked_against_every_other(lib):
    """A written tensor that overlaps any other tensor argument (inputs, parameters or another output)
    is refused with SSM_ERR_BAD_SHAPE before any HIP call."""
    assert scan(lib, last_state=OK_ARGS["B"] + 64) == SHAPE
    assert b"last_state" in lib.ssm_last_error_message()
    assert scan(lib, last_state=OK_ARGS["A"]) == SHAPE
    assert scan(lib, out=OK_ARGS["A"] + 256) == SHAPE
    assert scan(lib, D=P + 0x900000, out=P + 0x900000 - 64) == SHAPE   # out runs into D
    assert scan(lib, delta_bias=P + 0x500000 + 1024) == SHAPE          # bias inside out
    assert update(lib, state=P + 0x400000 + 32) == SHAPE               # state inside B
    assert update(lib, out=P + 0x300000) == SHAPE                      # out inside A
    assert bwd(lib, dA=P + 0x300000) == SHAPE                          # dA inside B
    assert bwd(lib, dD=P + 0x900000) == SHAPE                          # dD inside dB
    assert bwd(lib, dbias=P + 0x200000) == SHAPE                       # bias gradient inside A
    assert conv(lib, out=P + 0x100000) == SHAPE                        # out inside the weights
    assert window(lib, win=P + 0x200000) == SHAPE                      # window inside the weights


def ssd(lib, **kw):
    G = 1 << 30
    a = dict(x=P, a=P + G, b=P + 2 * G, c=P + 3 * G, y=P + 4 * G, fs=None, nb=2, L=100, H=8, Pd=64, N=128, ng=1, io=1,
             flags=0, ws=None, wsb=0)
    a.update(kw)
    return lib.ssm_ssd_scan(a["x"], a["a"], a["b"], a["c"], a["y"], a["fs"], a["nb"], a["L"], a["H"], a["Pd"], a["N"],
                            a["ng"], a["io"], a["flags"], a["ws"], a["wsb"], None)


def test_ssd_scan_validates(lib):
    """ssm_ssd_scan checks every argument before any HIP call."""
    for f in ("x", "a", "b", "c", "y"):
        assert ssd(lib, **{f: None}) == NULLP, f
    for kw in (dict(nb=0), dict(L=0), dict(H=0), dict(ng=0), dict(H=6, ng=4), dict(Pd=8), dict(Pd=80), dict(Pd=24),
               dict(N=0), dict(N=144), dict(N=20), dict(nb=1 << 40, L=1 << 40)):
        assert ssd(lib, **kw) == SHAPE, kw
    assert ssd(lib, io=2) == DTYPE
    assert ssd(lib, flags=FLAG_ZOH) == FLAGS
    assert ssd(lib, x=P + 8) == ALIGN
    assert ssd(lib, fs=P + 5 * (1 << 30) + 4) == ALIGN
    assert ssd(lib, y=P + 64) == SHAPE                       # y inside x
    assert ssd(lib, fs=P + 3 * (1 << 30) + 256) == SHAPE     # final state inside c
    assert b"headdim" in (ssd(lib, Pd=72) == SHAPE and lib.ssm_last_error_message())
    assert ssd(lib, L=(1 << 35) + 1, nb=1) == SHAPE


def test_ssd_workspace_size_and_checks(lib):
    """The workspace the split form takes: each segment's sum of a, then each segment's state (all but the
    last), rows padded to whole 16-state tiles; none where batch x heads fills the chip by itself."""
    sz = lib.ssm_ssd_scan_workspace_size
    # 4 x 80 heads (32-token chunks): 4 segments of 16 chunks; 3 stored states of 64 x 128 per head
    assert sz(4, 2048, 80, 64, 128, 1) == 320 * 4 * 4 + 320 * 3 * 64 * 128 * 4
    # 1 x 24 heads: 16 segments of 4 chunks
    assert sz(1, 2048, 24, 64, 128, 0) == 24 * 16 * 4 + 24 * 15 * 64 * 128 * 4
    # dstate 48 is kept as 64 columns; the decay sums round up to 256 bytes
    assert sz(1, 1000, 3, 16, 48, 1) == 256 + 3 * 15 * 16 * 64 * 4
    assert sz(1, 32, 3, 16, 48, 1) == 0           # one chunk: nothing to split
    assert sz(16, 4096, 64, 64, 128, 1) == 0      # 1024 (batch row, head) pairs fill the chip unsplit
    assert sz(0, 100, 8, 64, 128, 1) == 0 and sz(1, 100, 8, 64, 120, 1) == 0 and sz(1, 100, 8, 64, 128, 5) == 0
    need = sz(2, 100, 8, 64, 128, 1)
    W = P + 6 * (1 << 30)
    assert need > 0
    assert ssd(lib, ws=W, wsb=need - 1) == WSP
    assert b"ssm_ssd_scan_workspace_size" in lib.ssm_last_error_message()
    assert ssd(lib, ws=None, wsb=need) == WSP
    assert ssd(lib, ws=W + 8, wsb=need) == ALIGN
    assert ssd(lib, ws=P + 4 * (1 << 30) + 4096, wsb=need) == WSP   # inside y
    assert ssd(lib, ws=P - 256, wsb=need) == WSP                     # runs into x
