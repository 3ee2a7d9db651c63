"""Helpers for the GPU tests: move seeded numpy inputs to the device, run the HIP path through
the binding, bring results back as float64, and compare against the oracle elementwise."""
import numpy as np

import workloads as W

# Parity tolerances, elementwise |gpu - oracle| <= atol + rtol |oracle|: fp32 inputs -> rtol 1e-4 /
# atol 1e-5; bf16 inputs with fp32 state -> rtol 3e-3 / atol 1e-3 (oracle in fp64 on the same
# bf16-rounded inputs). They apply to fp32 results: the state, and the output before its cast. A bf16
# output is the final cast of that value (round to nearest even), which alone can move a value by up to
# 2^-8 of it (more than rtol 3e-3), so bf16 outputs are checked as the exact rounding of the fp32
# output of the same computation (assert_rounds_to), or, where the kernel has no fp32 output, as lying
# in the rounding of the tolerance interval (assert_close_before_cast).
TOL = {W.F32: (1e-4, 1e-5), W.BF16: (3e-3, 1e-3)}


def torch_mod():
    import torch

    return torch


def to_dev(a, device):
    if a is None:
        return None
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def from_dev(t):
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.double().cpu().numpy()


def assert_close(got, ref, io, what):
    """Elementwise |got - ref| <= atol + rtol |ref| at the tolerance of inputs of dtype `io`; `got` is
    an fp32 result (a state, or an output before its cast)."""
    rtol, atol = TOL[io]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values in the GPU result" % what
    lim = atol + rtol * np.abs(ref)
    err = np.abs(got - ref)
    bad = err > lim
    if bad.any():
        k = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError("%s: %d of %d elements outside rtol=%g atol=%g; worst at %s: gpu=%r oracle=%r"
                             % (what, int(bad.sum()), bad.size, rtol, atol, k, got[k], ref[k]))
    return float(err.max())


def bf16_round(x):
    """Round float64 values to bf16 (nearest even, via fp32) and return them as float64."""
    return W.bf16_bits_to_f64(W.to_io(np.asarray(x, dtype=np.float64), W.BF16))


def assert_rounds_to(got_bf16, got_f32, what):
    """A bf16 output is bit for bit the round-to-nearest-even of the fp32 output of the same call."""
    got_bf16 = np.asarray(got_bf16, dtype=np.float64)
    want = W.bf16_bits_to_f64(W.to_io(np.asarray(got_f32, dtype=np.float32).astype(np.float64), W.BF16))
    bad = got_bf16 != want
    if bad.any():
        k = np.unravel_index(np.argmax(bad), bad.shape)
        raise AssertionError("%s: %d of %d bf16 outputs are not the rounding of the fp32 output; first at %s: "
                             "bf16=%r fp32=%r" % (what, int(bad.sum()), bad.size, k, got_bf16[k], got_f32[k]))


def assert_close_before_cast(got_bf16, ref, io, what):
    """A bf16 output from a kernel without an fp32 output: it must be the rounding of some value within
    the tolerance of the oracle, i.e. lie between the roundings of the interval's ends (rounding is
    monotonic)."""
    rtol, atol = TOL[io]
    got = np.asarray(got_bf16, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lim = atol + rtol * np.abs(ref)
    lo, hi = bf16_round(ref - lim), bf16_round(ref + lim)
    bad = (got < lo) | (got > hi) | ~np.isfinite(got)
    if bad.any():
        k = np.unravel_index(np.argmax(bad), bad.shape)
        raise AssertionError("%s: %d of %d bf16 outputs outside the rounding of rtol=%g atol=%g; first at %s: "
                             "gpu=%r oracle=%r" % (what, int(bad.sum()), bad.size, rtol, atol, k, got[k], ref[k]))


def run_scan(inp, device, softplus=True, want_state=True, drop=(), zoh=False, out_f32=False):
    """Run the HIP scan on numpy inputs (io representation) and return float64 (out, last_state)."""
    import mamba_selective_scan_s6_amd as S

    t = {k: to_dev(inp.get(k), device) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    for k in drop:
        t[k] = None
    out, st = S.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                             softplus_flag=softplus, return_last_state=want_state, zoh=zoh, out_f32=out_f32)
    S.stream_check()  # synchronises; raises if a cross-workgroup wait in the kernel timed out
    return from_dev(out), (from_dev(st) if st is not None else None)


def run_oracle(inp, softplus=True, drop=(), channels=None, zoh=False):
    import oracle

    sub = W.rows_subset(inp, channels) if channels is not None else inp
    f = W.inputs_f64(sub)
    for k in drop:
        f[k] = None
    return oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"], f["delta_bias"],
                           softplus_flag=softplus, zoh=zoh)
