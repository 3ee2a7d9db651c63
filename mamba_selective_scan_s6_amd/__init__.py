"""mamba_selective_scan_s6_amd - the Mamba S6 selective scan on MI355X (gfx950).

A thin Python binding over the C ABI of ``libssmscan.so`` (declared in ``include/ssm_scan.h``).
It only marshals arguments: it checks torch tensors (device, dtype, shape, contiguity), passes
their device pointers and the current HIP stream, and raises on a nonzero status. Every step of
the computation runs in the HIP kernels; there is no fallback. If the library has not been built,
the first call raises.

    out, last_state = ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias, softplus_flag=True)
    out = ssm_state_update(state, x, delta, A, B, C, D, z)        # state updated in place

The scan kernels need a device workspace (the C ABI takes it from the caller). Unless a call passes
its own, the binding keeps one zero-filled torch buffer per (device, stream), grown when a larger
problem needs it; ``stream_check()`` reports a timed-out cross-workgroup wait on it.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["ssm_scan_fwd", "ssm_scan_bwd", "ssm_state_update", "causal_conv1d", "conv_window_update", "stream_check",
           "workspace_check", "release_workspaces", "scan_workspace_size", "scan_bwd_workspace_size", "set_wait_limit",
           "scan_segment_tokens", "ssd_scan", "ssd_workspace_size", "library_path", "load_library", "abi_version", "SSMError", "F32", "BF16", "FLAG_ZOH", "FLAG_OUT_F32"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssmscan.so")
_lock = threading.Lock()
_lib = None
_workspaces = {}  # (device index, raw stream handle) -> zero-filled uint8 tensor
_scratches = {}  # (device index, raw stream handle) -> uint8 tensor for ssm_ssd_scan

F32 = 0   # SSM_DTYPE_F32
BF16 = 1  # SSM_DTYPE_BF16
FLAG_ZOH = 1  # SSM_FLAG_ZOH: exact zero-order-hold input gain instead of the Euler gain
FLAG_OUT_F32 = 2  # SSM_FLAG_OUT_F32: fp32 output whatever the input dtype
MAX_DSTATE = 16


class SSMError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libssmscan.so (raises if it has not been built) and declare its signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libssmscan.so is not built; run `python -m mamba_selective_scan_s6_amd.build` "
                              "first (expected at %s)" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, fp, i64, ci = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.ssm_scan_fwd.restype = ci
        sz = ctypes.c_size_t
        lib.ssm_scan_fwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, ci, vp, fp, i64, i64, i64, i64, ci, vp, sz, vp]
        lib.ssm_scan_fwd_workspace_size.restype = sz
        lib.ssm_scan_fwd_workspace_size.argtypes = [i64, i64, i64]
        lib.ssm_scan_bwd_workspace_size.restype = sz
        lib.ssm_scan_bwd_workspace_size.argtypes = [i64, i64, i64]
        lib.ssm_state_update.restype = ci
        lib.ssm_state_update.argtypes = [fp, vp, vp, fp, vp, vp, fp, vp, vp, i64, i64, i64, ci, vp]
        cu = ctypes.c_uint
        lib.ssm_scan_fwd_ex.restype = ci
        lib.ssm_scan_fwd_ex.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, ci, vp, fp, i64, i64, i64, i64, ci, cu, vp, sz, vp]
        lib.ssm_state_update_ex.restype = ci
        lib.ssm_state_update_ex.argtypes = [fp, vp, vp, fp, vp, vp, fp, vp, vp, i64, i64, i64, ci, cu, vp]
        lib.ssm_scan_bwd.restype = ci
        lib.ssm_scan_bwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, ci, vp, vp, vp, fp, fp, fp, fp, vp, fp,
                                     i64, i64, i64, i64, ci, vp, sz, vp]
        lib.ssm_causal_conv1d.restype = ci
        lib.ssm_causal_conv1d.argtypes = [vp, fp, fp, ci, vp, i64, i64, i64, i64, ci, vp]
        lib.ssm_conv_window_update.restype = ci
        lib.ssm_conv_window_update.argtypes = [fp, vp, fp, fp, ci, vp, i64, i64, i64, ci, vp]
        lib.ssm_status_string.restype = ctypes.c_char_p
        lib.ssm_status_string.argtypes = [ci]
        lib.ssm_last_error_message.restype = ctypes.c_char_p
        lib.ssm_last_error_message.argtypes = []
        lib.ssm_abi_version.restype = ci
        lib.ssm_abi_version.argtypes = []
        lib.ssm_workspace_check.restype = ci
        lib.ssm_workspace_check.argtypes = [vp, vp]
        lib.ssm_ssd_scan.restype = ci
        lib.ssm_ssd_scan.argtypes = [vp, fp, vp, vp, vp, fp, i64, i64, i64, i64, i64, i64, ci, ctypes.c_uint, vp, sz,
                                     vp]
        lib.ssm_ssd_scan_workspace_size.restype = sz
        lib.ssm_ssd_scan_workspace_size.argtypes = [i64, i64, i64, i64, i64, ci]
        lib.ssm_set_wait_limit.restype = ci
        lib.ssm_set_wait_limit.argtypes = [ci]
        lib.ssm_scan_segment_tokens.restype = ci
        lib.ssm_scan_segment_tokens.argtypes = [i64, i64, i64]
        _lib = lib
        return lib


def abi_version() -> int:
    return load_library().ssm_abi_version()


def _check(lib, status: int):
    if status != 0:
        name = lib.ssm_status_string(status).decode()
        msg = lib.ssm_last_error_message().decode()
        raise SSMError(status, "%s: %s" % (name, msg))


def _io_code(t):
    import torch

    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("io tensors must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t, name, device, dtype=None, shape=None):
    if t is None:
        return None
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(device):
    import torch

    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)  # the handle alone, without a Stream object
    if raw is not None:
        return raw(device.index if device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def scan_workspace_size(batch: int, dim: int, seqlen: int) -> int:
    """Workspace bytes ssm_scan_fwd needs for these sizes (0 if they are invalid)."""
    return load_library().ssm_scan_fwd_workspace_size(batch, dim, seqlen)


def scan_bwd_workspace_size(batch: int, dim: int, seqlen: int) -> int:
    """Workspace bytes ssm_scan_bwd needs for these sizes (0 if they are invalid)."""
    return load_library().ssm_scan_bwd_workspace_size(batch, dim, seqlen)


def _workspace(need: int, device, workspace=None):
    """The caller's workspace if given (a CUDA uint8 tensor), else this (device, stream)'s cached one,
    replaced by a larger zero-filled buffer when `need` exceeds it. Returns (pointer, bytes)."""
    import torch

    if workspace is not None:
        if workspace.device != device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on %s" % device)
        return workspace.data_ptr(), workspace.numel() * workspace.element_size()
    key = (device.index if device.index is not None else torch.cuda.current_device(), _stream(device))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        # zero-filled once; the kernels leave it ready for the next call. A smaller buffer it
        # replaces is released in stream order by torch's allocator.
        ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws.data_ptr(), ws.numel()


def _scratch(need: int, device, workspace=None):
    """Like _workspace, for calls whose workspace needs no initialisation and keeps nothing between
    calls (ssm_ssd_scan): the caller's if given, else this (device, stream)'s cached one, grown as needed.
    Kept apart from the scan workspaces, whose contents must stay as the kernels left them."""
    import torch

    if workspace is not None:
        if workspace.device != device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on %s" % device)
        return workspace.data_ptr(), workspace.numel() * workspace.element_size()
    key = (device.index if device.index is not None else torch.cuda.current_device(), _stream(device))
    ws = _scratches.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1 << 20), dtype=torch.uint8, device=device)
        _scratches[key] = ws
    return ws.data_ptr(), ws.numel()


def ssm_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus_flag=True,
                 out=None, last_state=None, return_last_state=True, zoh=False, workspace=None, out_f32=False):
    """Selective scan forward on the current HIP stream.

    u, delta, z: [batch, dim, seqlen]; B, C: [batch, seqlen, dstate] (all float32, or all bfloat16);
    A: [dim, dstate] float32; D, delta_bias: [dim] float32 (optional). Returns (out, last_state)
    with out in u's dtype and last_state [batch, dim, dstate] float32 (None if not requested).
    zoh=True discretises the input with the exact zero-order hold instead of the Euler gain.
    workspace: optional caller-owned uint8 CUDA tensor of at least scan_workspace_size() bytes,
    zero-filled before its first use; by default the binding's cached one for this stream.
    out_f32=True writes out as float32 whatever the input dtype (the value a bf16 out is rounded from).
    """
    import torch

    lib = load_library()
    if u.dim() != 3:
        raise ValueError("u must be [batch, dim, seqlen]")
    nb, nd, L = u.shape
    if A.dim() != 2 or A.shape[0] != nd:
        raise ValueError("A must be [dim, dstate]")
    N = A.shape[1]
    dev, io = u.device, u.dtype
    code = _io_code(u)
    odt = torch.float32 if out_f32 else io
    if out is None:
        out = torch.empty(u.shape, dtype=odt, device=dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((nb, nd, N), dtype=torch.float32, device=dev)
    wsp, wsb = _workspace(lib.ssm_scan_fwd_workspace_size(nb, nd, L), dev, workspace)
    st = lib.ssm_scan_fwd_ex(
        _ptr(u, "u", dev, io), _ptr(delta, "delta", dev, io, (nb, nd, L)), _ptr(A, "A", dev, torch.float32),
        _ptr(B, "B", dev, io, (nb, L, N)), _ptr(C, "C", dev, io, (nb, L, N)),
        _ptr(D, "D", dev, torch.float32, (nd,)), _ptr(z, "z", dev, io, (nb, nd, L)),
        _ptr(delta_bias, "delta_bias", dev, torch.float32, (nd,)), int(bool(softplus_flag)),
        _ptr(out, "out", dev, odt, (nb, nd, L)), _ptr(last_state, "last_state", dev, torch.float32, (nb, nd, N)),
        nb, nd, L, N, code, (FLAG_ZOH if zoh else 0) | (FLAG_OUT_F32 if out_f32 else 0), wsp, wsb, _stream(dev))
    _check(lib, st)
    return out, last_state


def ssm_scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, dout=None, softplus_flag=True, workspace=None):
    """Gradients of ssm_scan_fwd (Euler input gain) for dout = dL/dout, on the current HIP stream.
    Returns a dict: du, ddelta, dz (like u; dz None without z), dA [dim, dstate], dB, dC [batch,
    seqlen, dstate], dD, ddelta_bias [dim] (float32; the gradient at 0 when the input was None)."""
    import torch

    lib = load_library()
    if u.dim() != 3:
        raise ValueError("u must be [batch, dim, seqlen]")
    nb, nd, L = u.shape
    N = A.shape[1]
    dev, io = u.device, u.dtype
    code = _io_code(u)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u), "dz": torch.empty_like(u) if z is not None else None,
         "dA": torch.empty((nd, N), **f32), "dB": torch.empty((nb, L, N), **f32), "dC": torch.empty((nb, L, N), **f32),
         "dD": torch.empty(nd, **f32), "ddelta_bias": torch.empty(nd, **f32)}
    wsp, wsb = _workspace(lib.ssm_scan_bwd_workspace_size(nb, nd, L), dev, workspace)
    st = lib.ssm_scan_bwd(
        _ptr(u, "u", dev, io), _ptr(delta, "delta", dev, io, (nb, nd, L)), _ptr(A, "A", dev, torch.float32, (nd, N)),
        _ptr(B, "B", dev, io, (nb, L, N)), _ptr(C, "C", dev, io, (nb, L, N)), _ptr(D, "D", dev, torch.float32, (nd,)),
        _ptr(z, "z", dev, io, (nb, nd, L)), _ptr(delta_bias, "delta_bias", dev, torch.float32, (nd,)),
        int(bool(softplus_flag)), _ptr(dout, "dout", dev, io, (nb, nd, L)), g["du"].data_ptr(), g["ddelta"].data_ptr(),
        g["dA"].data_ptr(), g["dB"].data_ptr(), g["dC"].data_ptr(), g["dD"].data_ptr(),
        g["dz"].data_ptr() if g["dz"] is not None else None, g["ddelta_bias"].data_ptr(), nb, nd, L, N, code,
        wsp, wsb, _stream(dev))
    _check(lib, st)
    return g


def workspace_check(workspace, device=None):
    """Synchronise the current stream and raise SSMError if a scan on `workspace` (a uint8 CUDA tensor)
    timed out waiting for another workgroup; the workspace is then zero-filled again."""
    import torch

    lib = load_library()
    dev = device if device is not None else workspace.device
    status = lib.ssm_workspace_check(workspace.data_ptr(), _stream(dev))
    if status != 0:
        workspace.zero_()
    _check(lib, status)


def stream_check(device=None):
    """Synchronise the current stream and raise SSMError if a scan on it (using the binding's cached
    workspace) timed out waiting for another workgroup (its outputs are invalid). Returns None when
    all is well."""
    import torch

    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    ws = _workspaces.get((dev.index if dev.index is not None else torch.cuda.current_device(), _stream(dev)))
    if ws is None:
        torch.cuda.current_stream(dev).synchronize()
        return
    workspace_check(ws, dev)


def scan_segment_tokens(batch: int, dim: int, seqlen: int) -> int:
    """Tokens per workgroup segment of the scan kernels (64)."""
    return load_library().ssm_scan_segment_tokens(batch, dim, seqlen)


def set_wait_limit(polls: int) -> int:
    """Polls a scan's cross-workgroup wait may take before it records a timeout (<= 0: default).
    Returns the previous limit."""
    return load_library().ssm_set_wait_limit(int(polls))


def release_workspaces():
    """Drop the binding's cached workspaces (the memory returns to torch's allocator)."""
    _workspaces.clear()
    _scratches.clear()


def ssm_state_update(state, x, delta, A, B, C, D=None, z=None, out=None, zoh=False, out_f32=False):
    """One decode step on the current HIP stream; ``state`` [batch, dim, dstate] float32 is updated
    in place. x, delta, z: [batch, dim]; B, C: [batch, dstate] (float32 or bfloat16); A: [dim, dstate]
    float32; D: [dim] float32. Returns out [batch, dim] in x's dtype. zoh=True: exact zero-order-hold
    input gain."""
    import torch

    lib = load_library()
    if state.dim() != 3:
        raise ValueError("state must be [batch, dim, dstate]")
    nb, nd, N = state.shape
    dev, io = x.device, x.dtype
    code = _io_code(x)
    odt = torch.float32 if out_f32 else io
    if out is None:
        out = torch.empty(x.shape, dtype=odt, device=dev)
    st = lib.ssm_state_update_ex(
        _ptr(state, "state", dev, torch.float32), _ptr(x, "x", dev, io, (nb, nd)),
        _ptr(delta, "delta", dev, io, (nb, nd)), _ptr(A, "A", dev, torch.float32, (nd, N)),
        _ptr(B, "B", dev, io, (nb, N)), _ptr(C, "C", dev, io, (nb, N)), _ptr(D, "D", dev, torch.float32, (nd,)),
        _ptr(z, "z", dev, io, (nb, nd)), _ptr(out, "out", dev, odt, (nb, nd)), nb, nd, N, code,
        (FLAG_ZOH if zoh else 0) | (FLAG_OUT_F32 if out_f32 else 0), _stream(dev))
    _check(lib, st)
    return out


def causal_conv1d(x, weight, bias=None, silu=True, out=None):
    """Causal depthwise convolution then SiLU on the current HIP stream. x: [batch, dim, seqlen]
    (float32 or bfloat16); weight: [dim, width] float32; bias: [dim] float32 (optional). Returns out
    like x."""
    import torch

    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [batch, dim, seqlen]")
    nb, nd, L = x.shape
    if weight.dim() != 2 or weight.shape[0] != nd:
        raise ValueError("weight must be [dim, width]")
    K = weight.shape[1]
    dev, io = x.device, x.dtype
    code = _io_code(x)
    if out is None:
        out = torch.empty_like(x)
    st = lib.ssm_causal_conv1d(_ptr(x, "x", dev, io), _ptr(weight, "weight", dev, torch.float32),
                               _ptr(bias, "bias", dev, torch.float32, (nd,)), int(bool(silu)),
                               _ptr(out, "out", dev, io, (nb, nd, L)), nb, nd, L, K, code, _stream(dev))
    _check(lib, st)
    return out


def conv_window_update(window, x, weight, bias=None, silu=True, out=None):
    """One decode step of the convolution on the current HIP stream; ``window`` [batch, dim, width]
    float32 (the last inputs, oldest first) is updated in place. x: [batch, dim]; weight: [dim,
    width] float32; bias: [dim] float32 (optional). Returns out like x."""
    import torch

    lib = load_library()
    if window.dim() != 3:
        raise ValueError("window must be [batch, dim, width]")
    nb, nd, K = window.shape
    dev, io = x.device, x.dtype
    code = _io_code(x)
    if out is None:
        out = torch.empty_like(x)
    st = lib.ssm_conv_window_update(_ptr(window, "window", dev, torch.float32), _ptr(x, "x", dev, io, (nb, nd)),
                                    _ptr(weight, "weight", dev, torch.float32, (nd, K)),
                                    _ptr(bias, "bias", dev, torch.float32, (nd,)), int(bool(silu)),
                                    _ptr(out, "out", dev, io, (nb, nd)), nb, nd, K, code, _stream(dev))
    _check(lib, st)
    return out


def ssd_workspace_size(batch: int, seqlen: int, heads: int, headdim: int, dstate: int, io_dtype: int) -> int:
    """Workspace bytes ssm_ssd_scan takes for these sizes (0: it runs unsplit and needs none)."""
    return load_library().ssm_ssd_scan_workspace_size(batch, seqlen, heads, headdim, dstate, io_dtype)


def ssd_scan(x, a, b, c, y=None, final_state=None, return_final_state=True, out_f32=False, workspace=None,
             split=True):
    """Mamba-2's scan with a scalar decay per head on the current HIP stream.

    x: [batch, seqlen, heads, headdim] (float32 or bfloat16; the stream already times its step);
    a: [batch, seqlen, heads] float32 (the step times A); b, c: [batch, seqlen, ngroups, dstate] in x's
    dtype. Returns (y [batch, seqlen, heads, headdim] in x's dtype, or float32 with out_f32=True;
    final_state [batch, heads, headdim, dstate] float32, or None when not requested).
    workspace: optional uint8 CUDA tensor of at least ssd_workspace_size() bytes; by default the binding
    keeps one per (device, stream). split=False passes no workspace: one workgroup per (batch row, head)
    walks the whole sequence.
    """
    import torch

    lib = load_library()
    if x.dim() != 4 or b.dim() != 4:
        raise ValueError("x must be [batch, seqlen, heads, headdim] and b, c [batch, seqlen, ngroups, dstate]")
    nb, L, H, P = x.shape
    G, N = b.shape[2], b.shape[3]
    dev, io = x.device, x.dtype
    code = _io_code(x)
    odt = torch.float32 if out_f32 else io
    if y is None:
        y = torch.empty((nb, L, H, P), dtype=odt, device=dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((nb, H, P, N), dtype=torch.float32, device=dev)
    wsa = (None, 0)
    if split:
        need = lib.ssm_ssd_scan_workspace_size(nb, L, H, P, N, code)
        if need or workspace is not None:
            wsa = _scratch(need, dev, workspace)
    st = lib.ssm_ssd_scan(_ptr(x, "x", dev, io), _ptr(a, "a", dev, torch.float32, (nb, L, H)),
                          _ptr(b, "b", dev, io, (nb, L, G, N)), _ptr(c, "c", dev, io, (nb, L, G, N)),
                          _ptr(y, "y", dev, odt, (nb, L, H, P)),
                          _ptr(final_state, "final_state", dev, torch.float32, (nb, H, P, N)),
                          nb, L, H, P, N, G, code, FLAG_OUT_F32 if out_f32 else 0, *wsa, _stream(dev))
    _check(lib, st)
    return y, final_state
