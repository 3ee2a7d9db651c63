"""fp64 CPU oracle for the Mamba S6 selective scan (test infrastructure only).

Only the tests, the smoke check and the benchmark's ``cpu_baseline`` leg may import this
package. The product path (the HIP library and its binding) never does, and the
two share no code: the oracle is plain C in ``oracle.c``, compiled by gcc without fast-math.

Functions follow the pages' definitions (see the header of ``oracle.c`` for the page titles
and sections): ``scan_fwd`` is the sequential loop of "Beyond attention with Mamba, state
space models and hybrids", section 4 (Mixer.forward with scan_loop), and ``state_update`` is
its section 7 one-token step; ``causal_conv1d`` and ``conv_window_update`` are the causal
convolution of "Module 19: State-Space Models (Mamba)" and section 7's window step; ``ssd_scan`` is
Mamba-2's scan with a scalar decay per head, the step-by-step loop of section 8. Inputs are numpy arrays of any float dtype; they are converted
to float64 (exact for float32 and for bfloat16 values) and results come back as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-pthread"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (IEEE fp64, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_softplus.restype = ctypes.c_double
    lib.oracle_softplus.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_scan_fwd.restype = ctypes.c_int
    lib.oracle_scan_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                    i64, i64, i64, i64, dp, dp, ctypes.c_int]
    lib.oracle_state_update.restype = ctypes.c_int
    lib.oracle_state_update.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int,
                                        i64, i64, i64, dp]
    lib.oracle_causal_conv1d.restype = ctypes.c_int
    lib.oracle_causal_conv1d.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, dp]
    lib.oracle_conv_window_update.restype = ctypes.c_int
    lib.oracle_conv_window_update.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                              ctypes.c_int64, dp]
    lib.oracle_scan_bwd.restype = ctypes.c_int
    lib.oracle_scan_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int, dp, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, dp, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_ssd_scan.restype = ctypes.c_int
    lib.oracle_ssd_scan.argtypes = [dp, dp, dp, dp, i64, i64, i64, i64, i64, i64, dp, dp, ctypes.c_int]
    lib.oracle_abi_version.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            _lib = _bind(_LIB)
        return _lib


def _f64(a, shape=None):
    if a is None:
        return None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and arr.shape != tuple(shape):
        arr = arr.reshape(shape)
    return arr


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    """Threads the oracle uses by default: the host's cores, capped by OMP_NUM_THREADS if set."""
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def softplus(r: float, _lib_override=None) -> float:
    return (_lib_override or _load()).oracle_softplus(float(r))


def silu(z: float, _lib_override=None) -> float:
    return (_lib_override or _load()).oracle_silu(float(z))


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus_flag=True, zoh=False,
             want_state=True, nthreads=None, _lib_override=None):
    """Selective scan. u, delta, z: [nb, nd, L]; B, C: [nb, L, N]; A: [nd, N]; D, delta_bias: [nd].

    Returns (out [nb, nd, L], last_state [nb, nd, N] or None), float64.
    """
    u = _f64(u)
    if u.ndim != 3:
        raise ValueError("u must be [batch, dim, seqlen]")
    nb, nd, L = u.shape
    A = _f64(A)
    N = A.shape[1]
    delta = _f64(delta, (nb, nd, L))
    B = _f64(B, (nb, L, N))
    C = _f64(C, (nb, L, N))
    D = _f64(D, (nd,))
    z = _f64(z, (nb, nd, L))
    delta_bias = _f64(delta_bias, (nd,))
    A = A.reshape(nd, N)
    out = np.empty((nb, nd, L), dtype=np.float64)
    last = np.empty((nb, nd, N), dtype=np.float64) if want_state else None
    rc = (_lib_override or _load()).oracle_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                 _ptr(delta_bias), int(bool(softplus_flag)), int(bool(zoh)),
                                 nb, nd, L, N, _ptr(out), _ptr(last),
                                 int(nthreads if nthreads is not None else default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_scan_fwd failed with code %d" % rc)
    return out, last


def state_update(state, x, delta, A, B, C, D=None, z=None, zoh=False, _lib_override=None):
    """One decode step. state: [nb, nd, N] (a float64 copy is updated and returned);
    x, delta, z: [nb, nd]; B, C: [nb, N]; A: [nd, N]; D: [nd].

    Returns (out [nb, nd], new_state [nb, nd, N]), float64.
    """
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    nb, nd, N = st.shape
    x = _f64(x, (nb, nd))
    delta = _f64(delta, (nb, nd))
    A = _f64(A, (nd, N))
    B = _f64(B, (nb, N))
    C = _f64(C, (nb, N))
    D = _f64(D, (nd,))
    z = _f64(z, (nb, nd))
    out = np.empty((nb, nd), dtype=np.float64)
    rc = (_lib_override or _load()).oracle_state_update(_ptr(st), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                     _ptr(D), _ptr(z), int(bool(zoh)), nb, nd, N, _ptr(out))
    if rc != 0:
        raise RuntimeError("oracle_state_update failed with code %d" % rc)
    return out, st


def scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, dout=None, softplus_flag=True, _lib_override=None):
    """Gradients of the selective scan (Euler input gain) given dout = dL/dout [nb, nd, L].

    Returns a dict of float64 arrays: du, ddelta [nb, nd, L]; dA [nd, N]; dB, dC [nb, L, N];
    dD, ddelta_bias [nd] (None when D / delta_bias are None); dz [nb, nd, L] (None when z is None).
    """
    u = _f64(u)
    nb, nd, L = u.shape
    A = _f64(A)
    N = A.shape[1]
    A = A.reshape(nd, N)
    delta = _f64(delta, (nb, nd, L))
    B = _f64(B, (nb, L, N))
    C = _f64(C, (nb, L, N))
    D = _f64(D, (nd,))
    z = _f64(z, (nb, nd, L))
    delta_bias = _f64(delta_bias, (nd,))
    dout = _f64(dout, (nb, nd, L))
    g = {"du": np.empty((nb, nd, L)), "ddelta": np.empty((nb, nd, L)), "dA": np.empty((nd, N)),
         "dB": np.empty((nb, L, N)), "dC": np.empty((nb, L, N)),
         "dD": np.empty(nd) if D is not None else None, "dz": np.empty((nb, nd, L)) if z is not None else None,
         "ddelta_bias": np.empty(nd) if delta_bias is not None else None}
    rc = (_lib_override or _load()).oracle_scan_bwd(
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), int(bool(softplus_flag)),
        _ptr(dout), nb, nd, L, N, _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
        _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddelta_bias"]))
    if rc != 0:
        raise RuntimeError("oracle_scan_bwd failed with code %d" % rc)
    return g


def causal_conv1d(x, w, bias=None, silu_flag=True, _lib_override=None):
    """Causal depthwise convolution (width K) then SiLU. x: [nb, nd, L]; w: [nd, K]; bias: [nd].
    Returns out [nb, nd, L], float64."""
    x = _f64(x)
    if x.ndim != 3:
        raise ValueError("x must be [batch, dim, seqlen]")
    nb, nd, L = x.shape
    w = _f64(w)
    K = w.shape[1]
    w = _f64(w, (nd, K))
    bias = _f64(bias, (nd,))
    out = np.empty((nb, nd, L), dtype=np.float64)
    rc = (_lib_override or _load()).oracle_causal_conv1d(_ptr(x), _ptr(w), _ptr(bias), int(bool(silu_flag)),
                                                         nb, nd, L, K, _ptr(out))
    if rc != 0:
        raise RuntimeError("oracle_causal_conv1d failed with code %d" % rc)
    return out


def conv_window_update(window, x, w, bias=None, silu_flag=True, _lib_override=None):
    """One decode step of the convolution. window: [nb, nd, K] (a float64 copy is updated and
    returned); x: [nb, nd]; w: [nd, K]; bias: [nd]. Returns (out [nb, nd], new_window)."""
    win = np.array(window, dtype=np.float64, copy=True, order="C")
    nb, nd, K = win.shape
    x = _f64(x, (nb, nd))
    w = _f64(w, (nd, K))
    bias = _f64(bias, (nd,))
    out = np.empty((nb, nd), dtype=np.float64)
    rc = (_lib_override or _load()).oracle_conv_window_update(_ptr(win), _ptr(x), _ptr(w), _ptr(bias),
                                                              int(bool(silu_flag)), nb, nd, K, _ptr(out))
    if rc != 0:
        raise RuntimeError("oracle_conv_window_update failed with code %d" % rc)
    return out, win


def ssd_scan(x, a, b, c, groups=None, want_state=True, nthreads=None, _lib_override=None):
    """Mamba-2's scan with a scalar decay per head (the step-by-step loop of "Beyond attention with
    Mamba, state space models and hybrids", section 8). x: [nb, L, heads, P] (already times the step);
    a: [nb, L, heads] (the step times A); b, c: [nb, L, groups, N] (a 3-d [nb, L, N] means one group).

    Returns (y [nb, L, heads, P], final_state [nb, heads, P, N] or None), float64.
    """
    x = _f64(x)
    if x.ndim != 4:
        raise ValueError("x must be [batch, seqlen, heads, headdim]")
    nb, L, H, P = x.shape
    b = _f64(b)
    if b.ndim == 3:
        b = b.reshape(nb, L, 1, b.shape[-1])
    G = b.shape[2] if groups is None else int(groups)
    N = b.shape[-1]
    b = _f64(b, (nb, L, G, N))
    c = _f64(c, (nb, L, G, N))
    a = _f64(a, (nb, L, H))
    y = np.empty((nb, L, H, P), dtype=np.float64)
    fin = np.empty((nb, H, P, N), dtype=np.float64) if want_state else None
    rc = (_lib_override or _load()).oracle_ssd_scan(_ptr(x), _ptr(a), _ptr(b), _ptr(c), nb, L, H, P, N, G, _ptr(y),
                                                    _ptr(fin), int(nthreads if nthreads is not None else default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_ssd_scan failed with code %d" % rc)
    return y, fin


class Variant:
    """The same API bound to another build of the oracle's C source (used by the tests that
    plant a mistake in a copy of the source and check that the pins catch it)."""

    def __init__(self, lib_path: str):
        self._lib = _bind(lib_path)

    def softplus(self, r):
        return softplus(r, _lib_override=self._lib)

    def silu(self, z):
        return silu(z, _lib_override=self._lib)

    def scan_fwd(self, *args, **kwargs):
        return scan_fwd(*args, _lib_override=self._lib, **kwargs)

    def state_update(self, *args, **kwargs):
        return state_update(*args, _lib_override=self._lib, **kwargs)

    def scan_bwd(self, *args, **kwargs):
        return scan_bwd(*args, _lib_override=self._lib, **kwargs)

    def causal_conv1d(self, *args, **kwargs):
        return causal_conv1d(*args, _lib_override=self._lib, **kwargs)

    def conv_window_update(self, *args, **kwargs):
        return conv_window_update(*args, _lib_override=self._lib, **kwargs)

    def ssd_scan(self, *args, **kwargs):
        return ssd_scan(*args, _lib_override=self._lib, **kwargs)


def build_variant(src_text: str, out_dir: str, name: str) -> str:
    """Compile C source text (a modified copy of oracle.c) into out_dir/name.so."""
    src = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", *CFLAGS, "-o", so, src, "-lm"])
    return so


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()
