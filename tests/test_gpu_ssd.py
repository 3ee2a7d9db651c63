"""GPU parity of the Mamba-2 scan (ssm_ssd_scan) against the fp64 oracle's step-by-step loop
("Beyond attention with Mamba, state space models and hybrids", section 8), elementwise.

Tolerance. Each output is a sum over earlier tokens and state numbers of terms of both signs,
(c_t . b_s) e^{a_{s+1}+...+a_t} x_s, many more of them than in the S6 scan (N = 128 and a window of
tokens), so where they cancel the result is known in fp32 only to a fraction of the terms' size, not of
its own. The bound is |gpu - oracle| <= atol + rtol |oracle| + kappa * magnitude, with the scan's rtol
and atol (fp32 inputs 1e-4 / 1e-5, bf16 inputs 3e-3 / 1e-3 on the fp32 output, SSM_FLAG_OUT_F32) and
magnitude = the sum of the terms' absolute values, which is the oracle itself run on |x|, |b|, |c| with
the same decays (every mask entry is positive). kappa = 1e-5 for fp32 inputs (about sqrt(K) times the
fp32 unit roundoff for the K ~ 10^4 terms of one output) and 3e-5 for bf16 inputs (the same, plus the
2^-17 left by splitting fp32 intermediates into two bf16 parts). The final state is checked the same way.
The bf16 output must be the round-to-nearest-even of the fp32 output. Heads are independent given the
inputs, so full-size shapes are checked on a sample of heads that the oracle computes alone."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import TOL, assert_close, assert_rounds_to, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import mamba_selective_scan_s6_amd as S

    S.load_library()
    return torch.device("cuda:0")


def run_ssd(inp, dev, out_f32=False, split=True):
    import mamba_selective_scan_s6_amd as S

    t = {k: to_dev(inp[k], dev) for k in ("x", "a", "b", "c")}
    y, fin = S.ssd_scan(t["x"], t["a"], t["b"], t["c"], out_f32=out_f32, split=split)
    return y, fin


KAPPA = {W.F32: 1e-5, W.BF16: 3e-5}


def oracle_ssd(inp, heads=None, magnitude=False):
    import oracle

    f = W.ssd_inputs_f64(inp)
    if heads is not None:
        f = dict(f, x=f["x"][:, :, heads], a=f["a"][:, :, heads])
    if magnitude:
        f = dict(f, x=np.abs(f["x"]), b=np.abs(f["b"]), c=np.abs(f["c"]))
    return oracle.ssd_scan(f["x"], f["a"], f["b"], f["c"])


def assert_close_cond(got, ref, mag, io, what):
    """assert_close's bound plus KAPPA[io] times the terms' magnitude."""
    rtol, atol = TOL[io]
    got, ref, mag = (np.asarray(v, dtype=np.float64) for v in (got, ref, mag))
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite values"
    lim = atol + rtol * np.abs(ref) + KAPPA[io] * mag
    err = np.abs(got - ref)
    bad = err > lim
    if bad.any():
        k = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError("%s: %d of %d outside; worst at %s: gpu=%r oracle=%r magnitude=%r"
                             % (what, int(bad.sum()), bad.size, k, got[k], ref[k], mag[k]))


def check_ssd(inp, dev, heads=None, what="ssd", split=True):
    io = inp["io"]
    y32, fin = run_ssd(inp, dev, out_f32=True, split=split)
    ref_y, ref_f = oracle_ssd(inp, heads)
    mag_y, mag_f = oracle_ssd(inp, heads, magnitude=True)
    gy, gf = from_dev(y32), from_dev(fin)
    if heads is not None:
        gy, gf = gy[:, :, heads], gf[:, heads]
    assert_close_cond(gy, ref_y, mag_y, io, what + " y")
    assert_close_cond(gf, ref_f, mag_f, io, what + " final state")
    if io == W.BF16:
        y16, _ = run_ssd(inp, dev, split=split)
        assert_rounds_to(from_dev(y16), from_dev(y32), what + " bf16 y")


SHAPES = [  # nb, L, H, P, N, G
    (1, 150, 3, 16, 16, 3),     # section 8's check, with P and N raised to the kernel's 16
    (2, 77, 4, 32, 32, 2),      # ragged chunk, groups of two heads
    (1, 1, 2, 16, 16, 1),       # one token
    (1, 32, 1, 64, 128, 1),     # exactly one chunk
    (1, 64, 1, 64, 128, 1),     # exactly two chunks
    (1, 65, 2, 48, 64, 1),      # one token past two chunks
    (2, 200, 6, 64, 128, 3),    # several chunks, three groups
    (1, 33, 5, 16, 112, 5),     # every head its own b and c
]


@pytest.mark.parametrize("io", [W.F32, W.BF16])
@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
def test_ssd_small_shapes(dev, shape, io):
    nb, L, H, P, N, G = shape
    for layer in (True, False):
        inp = W.make_ssd_inputs(nb, L, H, P, N, G, io, seed=sum(shape) + (7 if layer else 0), layer=layer)
        for split in (True, False):
            check_ssd(inp, dev, what="%s %s layer=%s split=%s" % (shape, io, layer, split), split=split)


SPLIT_SHAPES = [  # nb, L, H, P, N, G: few (batch row, head) pairs, so the sequence is cut into segments
    (1, 1000, 3, 16, 48, 1),    # 16 segments of two chunks; dstate padded to 64 columns in the carries
    (1, 700, 2, 64, 128, 2),    # 11 segments of two chunks, the last ragged
    (2, 4096, 4, 32, 64, 1),    # long segments (8 chunks each)
    (1, 65, 1, 16, 16, 1),      # three one-chunk segments, the last one token long
]


@pytest.mark.parametrize("io", [W.F32, W.BF16])
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=["x".join(map(str, s)) for s in SPLIT_SHAPES])
def test_ssd_segments(dev, shape, io):
    """The split form (segment states, their carries, then every segment's outputs in parallel) against
    the oracle, and against the unsplit walk: the same values up to rounding."""
    import mamba_selective_scan_s6_amd as S

    nb, L, H, P, N, G = shape
    code = S.BF16 if io == W.BF16 else S.F32
    assert S.ssd_workspace_size(nb, L, H, P, N, code) > 0, "shape does not split"
    inp = W.make_ssd_inputs(nb, L, H, P, N, G, io, seed=L + H)
    check_ssd(inp, dev, what="%s %s split" % (shape, io))
    ys, fs = (from_dev(v) for v in run_ssd(inp, dev, out_f32=True))
    yu, fu = (from_dev(v) for v in run_ssd(inp, dev, out_f32=True, split=False))
    mag_y, mag_f = oracle_ssd(inp, magnitude=True)
    assert_close_cond(ys, yu, mag_y, io, "split vs unsplit y")
    assert_close_cond(fs, fu, mag_f, io, "split vs unsplit final state")


@pytest.mark.parametrize("cfg_id,heads", [("ssd130m", [0, 11, 23]), ("ssd2p7b", [0, 41, 79])])
def test_ssd_full_size_sampled(dev, cfg_id, heads):
    """The benchmark's shapes at full size, in the launch it times; the oracle computes three heads."""
    inp = W.make_ssd_config_inputs(W.SSD_CONFIGS[cfg_id])
    check_ssd(inp, dev, heads=heads, what=cfg_id)


def test_ssd_strong_and_no_decay(dev):
    """Decays that forget everything within a token (a = -60) and none at all (a = 0) over several chunks."""
    for av in (-60.0, 0.0):
        inp = W.make_ssd_inputs(1, 300, 2, 32, 64, 1, W.F32, seed=5, layer=False)
        inp["a"] = np.full_like(inp["a"], av)
        inp["x"] = (0.1 * inp["x"]).astype(np.float32)
        check_ssd(inp, dev, what="a=%g" % av)


def test_ssd_run_to_run_bitwise(dev):
    inp = W.make_ssd_inputs(2, 300, 4, 64, 128, 1, W.BF16, seed=9)
    y1, f1 = run_ssd(inp, dev)
    y2, f2 = run_ssd(inp, dev)
    import torch

    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_ssd_matches_the_s6_scan_when_a_is_shared(dev):
    """With headdim 16 channels that each carry the same step, and A equal across state numbers, each
    channel of a head is an S6 scan (softplus off, no skip, no gate) on the GPU too."""
    import mamba_selective_scan_s6_amd as S
    import torch

    rng = np.random.default_rng(21)
    nb, L, H, P, N = 1, 130, 2, 16, 16
    u = rng.standard_normal((nb, L, H, P)).astype(np.float32)
    dt = rng.uniform(0.01, 0.3, size=(nb, L, H)).astype(np.float32)
    Ah = -rng.uniform(0.2, 2.0, size=H).astype(np.float32)
    B = rng.standard_normal((nb, L, 1, N)).astype(np.float32)
    C = rng.standard_normal((nb, L, 1, N)).astype(np.float32)
    x = (u * dt[..., None]).astype(np.float32)
    a = (dt * Ah).astype(np.float32)
    y, fin = S.ssd_scan(*(to_dev(v, dev) for v in (x, a, B, C)))
    # the same as S6 scans: channel (h, p) with delta = dt[h] broadcast, A[n] = Ah[h], u = u[.., h, p]
    us = np.ascontiguousarray(u.transpose(0, 2, 3, 1).reshape(nb, H * P, L))
    ds = np.ascontiguousarray(np.repeat(dt.transpose(0, 2, 1), P, axis=1))
    As = np.repeat(np.repeat(Ah[:, None], P, axis=0), N, axis=1).astype(np.float32)
    out, last = S.ssm_scan_fwd(to_dev(us, dev), to_dev(ds, dev), to_dev(As, dev), to_dev(B[:, :, 0], dev),
                               to_dev(C[:, :, 0], dev), softplus_flag=False)
    torch.cuda.synchronize()
    got = from_dev(y).transpose(0, 2, 3, 1).reshape(nb, H * P, L)
    assert_close(got, from_dev(out), W.F32, "ssd vs s6 y")
    assert_close(from_dev(fin).reshape(nb, H * P, N), from_dev(last), W.F32, "ssd vs s6 state")


def test_ssd_caller_workspace_and_reuse(dev):
    """A caller-owned workspace gives the binding's result bit for bit, and keeps nothing between calls:
    a larger problem, then a smaller one on the same workspace, each match a fresh call."""
    import mamba_selective_scan_s6_amd as S
    import torch

    shapes = [(2, 900, 3, 64, 128, 1), (1, 130, 2, 16, 32, 2)]
    need = max(S.ssd_workspace_size(nb, L, H, P, N, S.BF16) for nb, L, H, P, N, _ in shapes)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    for nb, L, H, P, N, G in shapes:
        inp = W.make_ssd_inputs(nb, L, H, P, N, G, W.BF16, seed=L)
        t = [to_dev(inp[k], dev) for k in ("x", "a", "b", "c")]
        y1, f1 = S.ssd_scan(*t, workspace=ws, out_f32=True)
        y2, f2 = S.ssd_scan(*t, out_f32=True)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(f1, f2), (nb, L, H, P, N, G)
    small = torch.empty(max(need // 2, 256), dtype=torch.uint8, device=dev)
    inp = W.make_ssd_inputs(*shapes[0], W.BF16, seed=1)
    with pytest.raises(S.SSMError):
        S.ssd_scan(*(to_dev(inp[k], dev) for k in ("x", "a", "b", "c")), workspace=small)

