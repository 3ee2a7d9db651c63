"""Helpers for the GPU tests: move seeded numpy inputs to the device, run the HIP path through
the binding, bring results back as float64, and compare against the oracle elementwise."""
import numpy as np

import workloads as W

# Parity tolerances: fp32 io -> rtol 1e-4 / atol 1e-5; bf16 io with fp32 state -> rtol 3e-3 /
# atol 1e-3 (oracle in fp64 on the same bf16-rounded inputs). A bf16 output is additionally
# rounded to nearest even by the final cast, which adds up to half a bf16 ulp of the value.
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


def half_ulp_bf16(x):
    """Half a bf16 ulp at |x| (bf16 keeps 8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(np.where(ax > 0, ax, 1.0))  # ax = m * 2^e, m in [0.5, 1)
    return np.where(ax > 0, np.ldexp(1.0, e - 1 - 8), 0.0)


def assert_close(got, ref, io, what, output_cast=True):
    rtol, atol = TOL[io]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values in the GPU result" % what
    lim = atol + rtol * np.abs(ref)
    if io == W.BF16 and output_cast:
        lim = lim + half_ulp_bf16(ref)
    err = np.abs(got - ref)
    bad = err > lim
    if bad.any():
        k = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError("%s: %d of %d elements outside rtol=%g atol=%g; worst at %s: gpu=%r oracle=%r"
                             % (what, int(bad.sum()), bad.size, rtol, atol, k, got[k], ref[k]))
    return float(err.max())


def run_scan(inp, device, softplus=True, want_state=True, drop=(), zoh=False):
    """Run the HIP scan on numpy inputs (io representation) and return float64 (out, last_state)."""
    import mamba_selective_scan_s6_amd as S

    t = {k: to_dev(inp.get(k), device) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    for k in drop:
        t[k] = None
    out, st = S.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"],
                             softplus_flag=softplus, return_last_state=want_state, zoh=zoh)
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
