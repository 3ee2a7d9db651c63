"""The scan entry point that allocates nothing (ssm_scan_fwd_noalloc), called through the C ABI: its
output and final state equal those of ssm_scan_fwd (the same kernels, on the library's own device
array instead of a caller's workspace) bit for bit, on two calls in a row, the second with a smaller
input. (Its refusal of problems beyond the array is checked on the host, in test_abi_host.py.)"""
import ctypes

import numpy as np
import pytest

import workloads as W
from gpu_helpers import from_dev, to_dev

pytestmark = pytest.mark.gpu

FLAG_OUT_F32 = 2


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import mamba_selective_scan_s6_amd as S

    S.load_library()
    return torch.device("cuda:0")


def _lib():
    import mamba_selective_scan_s6_amd as S

    lib = S.load_library()
    vp, fp, i64, ci, cu = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint
    lib.ssm_scan_fwd_noalloc.restype = ci
    lib.ssm_scan_fwd_noalloc.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, ci, vp, fp, i64, i64, i64, i64, ci, cu, vp]
    lib.ssm_scan_fwd_noalloc_max_workspace.restype = ctypes.c_size_t
    lib.ssm_scan_fwd_noalloc_max_workspace.argtypes = []
    return lib


def _noalloc(t, out, st, io, flags=0):
    import torch

    nb, nd, L = t["u"].shape
    N = t["A"].shape[1]
    p = lambda x: x.data_ptr() if x is not None else None  # noqa: E731
    code = 1 if io == W.BF16 else 0
    stream = torch.cuda.current_stream().cuda_stream
    return _lib().ssm_scan_fwd_noalloc(p(t["u"]), p(t["delta"]), p(t["A"]), p(t["B"]), p(t["C"]), p(t["D"]), p(t["z"]),
                                       p(t["delta_bias"]), 1, p(out), p(st), nb, nd, L, N, code, flags, stream)


def test_noalloc_matches_the_workspace_entry_point(dev):
    import mamba_selective_scan_s6_amd as S
    import torch

    problems = [W.make_scan_inputs(2, 200, 700, 16, W.BF16, seed=301),   # 2 x 4 x 11 segments
                W.make_scan_inputs(1, 64, 130, 16, W.F32, seed=302)]     # then a smaller one
    for inp in problems:
        t = {k: to_dev(inp.get(k), dev) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
        nb, nd, L = t["u"].shape
        for flags in ((0, FLAG_OUT_F32) if inp["io"] == W.BF16 else (0,)):
            odt = torch.float32 if flags & FLAG_OUT_F32 else t["u"].dtype
            out = torch.empty((nb, nd, L), dtype=odt, device=dev)
            st = torch.empty((nb, nd, 16), dtype=torch.float32, device=dev)
            assert _noalloc(t, out, st, inp["io"], flags) == 0, _lib().ssm_last_error_message()
            ref_out, ref_st = S.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                                             out_f32=bool(flags & FLAG_OUT_F32))
            torch.cuda.synchronize()
            np.testing.assert_array_equal(from_dev(out), from_dev(ref_out))
            np.testing.assert_array_equal(from_dev(st), from_dev(ref_st))
