"""GPU parity of the backward scan (ssm_scan_bwd) against the fp64 oracle's backward, which the CPU
pins tie to finite differences of the forward oracle.

Elementwise gradients (du, ddelta, dz: one value per batch row, channel and token) meet the forward's
tolerance for the input dtype, elementwise: fp32 io rtol 1e-4 / atol 1e-5; bf16 io rtol 3e-3 /
atol 1e-3, applied before the final bf16 cast (the stored bf16 value must be the rounding of a value
within the tolerance). The sums (dA, dD and the bias gradient over batch rows and tokens; dB, dC over
channels) take an atol scaled by the array's largest entry, at the same rtol: each is a sum of
thousands of terms of both signs, summed in a different order than the oracle's, so an entry whose
terms cancel is known only to a fraction of the terms' size, not of its own."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import TOL, assert_close, assert_close_before_cast, from_dev, to_dev

pytestmark = pytest.mark.gpu

ELEMENTWISE = ("du", "ddelta", "dz")
SUMS = ("dA", "dB", "dC", "dD", "ddelta_bias")


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import mamba_selective_scan_s6_amd as S

    S.load_library()
    return torch.device("cuda:0")


def _close_sum(got, ref, io, what):
    rtol, _ = TOL[io]
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite"
    lim = rtol * np.abs(ref) + rtol * max(float(np.max(np.abs(ref))), 1e-30)
    bad = np.abs(got - ref) > lim
    if bad.any():
        k = np.unravel_index(np.argmax(np.abs(got - ref) - lim), got.shape)
        raise AssertionError("%s: %d of %d outside; worst at %s gpu=%r ref=%r" % (what, int(bad.sum()), bad.size, k,
                                                                               got[k], ref[k]))


def check_bwd(inp, dev, softplus=True, drop=(), seed=0):
    import mamba_selective_scan_s6_amd as S
    import oracle

    io = inp["io"]
    rng = np.random.default_rng(seed)
    dout = W.to_io(rng.standard_normal(inp["u"].shape), io)
    t = {k: to_dev(inp.get(k), dev) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    for k in drop:
        t[k] = None
    g = S.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                       dout=to_dev(dout, dev), softplus_flag=softplus)
    S.stream_check()
    f = W.inputs_f64(inp)
    for k in drop:
        f[k] = None
    ref = oracle.scan_bwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"], f["delta_bias"],
                          dout=W.io_to_f64(dout, io), softplus_flag=softplus)
    for name in ELEMENTWISE + SUMS:
        if ref[name] is None:
            continue
        if name in SUMS:
            _close_sum(from_dev(g[name]), ref[name], io, name)
        elif io == W.F32:
            assert_close(from_dev(g[name]), ref[name], io, name)
        else:
            assert_close_before_cast(from_dev(g[name]), ref[name], io, name)


@pytest.mark.parametrize("nb,nd,L,N,io", [(1, 64, 16, 16, W.F32), (2, 70, 50, 16, W.F32), (1, 130, 300, 16, W.BF16),
                                          (2, 100, 77, 5, W.F32), (1, 33, 7, 16, W.BF16), (1, 20, 1, 16, W.F32),
                                          (2, 256, 1000, 16, W.F32), (3, 64, 129, 3, W.BF16)])
def test_scan_bwd_parity(dev, nb, nd, L, N, io):
    inp = W.make_scan_inputs(nb, nd, L, N, io, seed=1000 + nb + nd + L + N)
    check_bwd(inp, dev, seed=L)


@pytest.mark.parametrize("drop", [("D",), ("z",), ("delta_bias",), ("D", "z", "delta_bias")])
def test_scan_bwd_optional_inputs(dev, drop):
    inp = W.make_scan_inputs(2, 96, 130, 16, W.F32, seed=1077)
    check_bwd(inp, dev, drop=drop, seed=3)


def test_scan_bwd_softplus_off(dev):
    inp = W.make_scan_inputs(2, 80, 90, 16, W.F32, seed=1078)
    inp["delta"] = (np.abs(inp["delta"]) * 0.2).astype(np.float32)
    inp["delta_bias"] = np.full(80, 0.01, np.float32)
    check_bwd(inp, dev, softplus=False, seed=4)


def test_scan_bwd_is_reproducible(dev):
    import mamba_selective_scan_s6_amd as S

    inp = W.make_scan_inputs(2, 200, 700, 16, W.BF16, seed=1079)
    dout = to_dev(W.to_io(np.random.default_rng(5).standard_normal(inp["u"].shape), W.BF16), dev)
    t = {k: to_dev(inp.get(k), dev) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    g1 = S.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], dout=dout)
    g2 = S.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], dout=dout)
    for k in g1:
        np.testing.assert_array_equal(from_dev(g1[k]), from_dev(g2[k]), err_msg=k)
