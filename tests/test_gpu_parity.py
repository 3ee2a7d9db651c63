"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element, on the
same seeded inputs. Small shapes run the oracle on everything; the full-size workloads run the
GPU on everything and the oracle on sampled channels (rows are independent, so the oracle's rows
are exact references for those channels)."""
import math
import sys

import numpy as np
import pytest

import workloads as W
from conftest import golden
from gpu_helpers import assert_close, assert_close_before_cast, assert_rounds_to, from_dev, run_oracle, run_scan, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write("[gpu-test] %s\n" % request.node.nodeid)
    sys.__stderr__.flush()
    yield


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import mamba_selective_scan_s6_amd as S

    S.load_library()  # raises if the HIP library is missing: no silent fallback
    return torch.device("cuda:0")


def check_scan(inp, dev, channels=None, softplus=True, drop=(), what="", zoh=False):
    """The scan against the oracle. The fp32 output (with bf16 inputs: SSM_FLAG_OUT_F32, the value the
    bf16 output is rounded from) and the final state meet the tolerance of the input dtype; with bf16
    inputs the default bf16 output is then, bit for bit, the rounding of that fp32 output."""
    drop_in = tuple(d for d in drop if d != "last_state")
    want_state = "last_state" not in drop
    ref_out, ref_st = run_oracle(inp, softplus=softplus, drop=drop_in, channels=channels, zoh=zoh)
    out, st = run_scan(inp, dev, softplus=softplus, drop=drop_in, want_state=want_state, zoh=zoh, out_f32=True)
    sel = (lambda a: a[:, channels]) if channels is not None else (lambda a: a)
    e1 = assert_close(sel(out), ref_out, inp["io"], what + " out")
    if want_state:
        assert_close(sel(st), ref_st, inp["io"], what + " last_state")
    if inp["io"] == W.BF16:
        out16, st16 = run_scan(inp, dev, softplus=softplus, drop=drop_in, want_state=want_state, zoh=zoh)
        assert_rounds_to(out16, out, what + " bf16 out")
        if want_state:
            np.testing.assert_array_equal(st16, st)
    return e1


def decode_step(state, t, A, D, z, check_bf16=False, zoh=False):
    """One decode update with fp32 output (returned); with check_bf16 the same step also runs with the
    default bf16 output on a copy of the state, which must end equal and whose output must be the
    rounding of the fp32 one."""
    import mamba_selective_scan_s6_amd as S
    import torch

    if check_bf16:
        st2 = state.clone()
        o16 = S.ssm_state_update(st2, t["x"], t["delta"], A, t["B"], t["C"], D, z, zoh=zoh)
    o32 = S.ssm_state_update(state, t["x"], t["delta"], A, t["B"], t["C"], D, z, zoh=zoh, out_f32=True)
    if check_bf16:
        torch.cuda.synchronize()
        assert_rounds_to(from_dev(o16), from_dev(o32), "decode bf16 out")
        assert torch.equal(st2, state)
    return o32


# ---------------------------------------------------------------- whole-tensor parity, small shapes
def test_toy_config_full(dev):
    cfg = W.SCAN_CONFIGS["toy"]
    check_scan(W.make_config_inputs(cfg), dev, what=cfg.name)


@pytest.mark.parametrize("nb,nd,L,io", [(2, 100, 77, W.F32), (3, 130, 300, W.BF16), (1, 1, 1, W.F32),
                                        (1, 65, 513, W.BF16), (2, 64, 1000, W.F32), (1, 192, 2049, W.BF16),
                                        (1, 7, 5, W.BF16)])
def test_small_shapes(dev, nb, nd, L, io):
    inp = W.make_scan_inputs(nb, nd, L, 16, io, seed=nb * 1000 + nd + L)
    check_scan(inp, dev, what="%dx%dx%d %s" % (nb, nd, L, io))


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8, 15, 16])
@pytest.mark.parametrize("io", [W.F32, W.BF16])
def test_dstate_values(dev, N, io):
    inp = W.make_scan_inputs(2, 70, 50, N, io, seed=40 + N)
    check_scan(inp, dev, what="N=%d %s" % (N, io))


@pytest.mark.parametrize("drop", [("D",), ("z",), ("delta_bias",), ("last_state",), ("D", "z", "delta_bias")])
@pytest.mark.parametrize("io", [W.F32, W.BF16])
def test_optional_inputs(dev, drop, io):
    inp = W.make_scan_inputs(1, 96, 130, 16, io, seed=77)
    check_scan(inp, dev, drop=drop, what="without %s" % (drop,))


def test_softplus_off(dev):
    inp = W.make_scan_inputs(2, 80, 90, 16, W.F32, seed=78)
    inp["delta"] = (np.abs(inp["delta"]) * 0.2).astype(np.float32)  # a positive step without softplus
    inp["delta_bias"] = np.full(80, 0.01, np.float32)
    check_scan(inp, dev, softplus=False, what="softplus off")


# ---------------------------------------------------------------- full-size workloads, sampled rows
def _sample_channels(nd, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 127, nd // 2, nd - 65, nd - 64, nd - 1]
    extra = rng.choice(nd, size=8, replace=False).tolist()
    return sorted(set(c for c in fixed + extra if 0 <= c < nd))


@pytest.mark.parametrize("cfg_id", ["mamba130m", "mamba2p8b", "long"])
def test_full_size_config_sampled(dev, cfg_id):
    cfg = W.SCAN_CONFIGS[cfg_id]
    inp = W.make_config_inputs(cfg)
    ch = _sample_channels(cfg.nd, cfg.seed)
    check_scan(inp, dev, channels=ch, what=cfg.name)


# ---------------------------------------------------------------- larger shapes, sampled channels
# Edge cases at sizes with many segments and channel groups in flight at once.
@pytest.mark.parametrize("nb,nd,L,N,io", [(4, 2048, 2050, 16, W.F32),     # ragged L, scalar loads
                                          (2, 4100, 1024, 5, W.BF16),     # ragged channel group, N < 16
                                          (4, 2048, 2047, 16, W.BF16)])   # ragged L, bf16
def test_many_groups_sampled(dev, nb, nd, L, N, io):
    inp = W.make_scan_inputs(nb, nd, L, N, io, seed=nd + L + N)
    check_scan(inp, dev, channels=_sample_channels(nd, L), what="%dx%dx%d N%d %s" % (nb, nd, L, N, io))


def test_many_groups_optional_inputs_softplus_off(dev):
    nb, nd, L = 2, 4096, 1024
    inp = W.make_scan_inputs(nb, nd, L, 16, W.F32, seed=91)
    inp["delta"] = (np.abs(inp["delta"]) * 0.2).astype(np.float32)  # a positive step without softplus
    check_scan(inp, dev, channels=_sample_channels(nd, 91), softplus=False, drop=("D", "z", "delta_bias"),
               what="2x4096x1024 without D, z, bias, softplus off")


def test_many_groups_run_to_run_bitwise(dev):
    nb, nd, L = 4, 2048, 2050
    inp = W.make_scan_inputs(nb, nd, L, 16, W.BF16, seed=92)
    o1, s1 = run_scan(inp, dev)
    o2, s2 = run_scan(inp, dev)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


# ---------------------------------------------------------------- properties
@pytest.mark.parametrize("io", [W.F32, W.BF16])
@pytest.mark.parametrize("field", ["u", "delta", "z", "B", "C"])
def test_causality_bitwise(dev, io, field):
    inp = W.make_scan_inputs(1, 128, 200, 16, io, seed=5)
    out1, _ = run_scan(inp, dev)
    t = 137
    mod = dict(inp)
    arr = inp[field].copy()
    if field in ("B", "C"):
        arr[:, t, :] = arr[:, t, ::-1]
    else:
        arr[:, :, t] = arr[:, ::-1, t]
    mod[field] = arr
    out2, _ = run_scan(mod, dev)
    np.testing.assert_array_equal(out1[:, :, :t], out2[:, :, :t])
    assert np.any(out1[:, :, t] != out2[:, :, t])


def test_run_to_run_bitwise(dev):
    inp = W.make_config_inputs(W.SCAN_CONFIGS["mamba130m"])
    o1, s1 = run_scan(inp, dev)
    o2, s2 = run_scan(inp, dev)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_softplus_accuracy(dev):
    """With A = 0, B = C = 1, u = 1 and one token, out equals the step Delta = softplus(delta):
    the kernel's softplus against the oracle's over [-20, 20]."""
    import oracle

    nd = 4096
    r = np.linspace(-20.0, 20.0, nd).astype(np.float32)
    inp = dict(u=np.ones((1, nd, 1), np.float32), delta=r.reshape(1, nd, 1), A=np.zeros((nd, 1), np.float32),
               B=np.ones((1, 1, 1), np.float32), C=np.ones((1, 1, 1), np.float32), D=None, z=None,
               delta_bias=None, io=W.F32)
    out, _ = run_scan(inp, dev)
    ref = np.array([oracle.softplus(float(x)) for x in r])
    np.testing.assert_allclose(out.reshape(-1), ref, rtol=2e-6, atol=0)


def test_page_toys_on_gpu(dev):
    """The printed worked examples, run on the GPU through the C ABI (N = 1)."""
    g = golden("p5_toy_recurrence.json")
    inp = dict(u=np.array([[g["inputs"]]], np.float32), delta=np.ones((1, 1, 4), np.float32),
               A=np.array([[math.log(g["Abar"])]], np.float32), B=np.full((1, 4, 1), g["Bbar"], np.float32),
               C=np.ones((1, 4, 1), np.float32), D=None, z=None, delta_bias=None, io=W.F32)
    out, st = run_scan(inp, dev, softplus=False)
    assert np.round(out.reshape(-1), g["decimals"]).tolist() == g["states"]
    g = golden("m19_parallel_scan.json")
    a, b = np.array(g["a"]), np.array(g["b"])
    dt = -np.log(a)
    inp = dict(u=np.ones((1, 1, 5), np.float32), delta=dt.reshape(1, 1, 5).astype(np.float32),
               A=np.array([[-1.0]], np.float32), B=(b / dt).reshape(1, 5, 1).astype(np.float32),
               C=np.ones((1, 5, 1), np.float32), D=None, z=None, delta_bias=None, io=W.F32)
    out, _ = run_scan(inp, dev, softplus=False)
    np.testing.assert_allclose(out.reshape(-1), g["h"], atol=6e-5)


def test_degenerate_steps(dev):
    """Delta = 0 leaves the state untouched (out = D u SiLU(z)); a huge step resets it."""
    inp = W.make_scan_inputs(1, 64, 40, 16, W.F32, seed=9)
    inp["delta"] = np.zeros_like(inp["delta"])
    out, st = run_scan(inp, dev, softplus=False, drop=("delta_bias",))
    x = inp["u"].astype(np.float64)
    z = inp["z"].astype(np.float64)
    expect = inp["D"].astype(np.float64)[None, :, None] * x * z / (1 + np.exp(-z))
    np.testing.assert_allclose(out, expect, rtol=1e-5, atol=1e-6)
    assert np.all(st == 0)
    inp2 = W.make_scan_inputs(1, 64, 40, 16, W.F32, seed=10)
    inp2["delta"][:, :, 20] = 80.0  # exp(80 * A) underflows: the state restarts at token 20
    check_scan(inp2, dev, what="reset step")


# ---------------------------------------------------------------- decode
def _decode_inputs_dev(step_inp, dev):
    return {k: to_dev(v, dev) for k, v in step_inp.items()}


def test_decode_config_sampled(dev):
    """256 decode steps on the persistent [64, 8192, 16] state; the oracle follows sampled channels
    (every batch row) in fp64 from the same fp32 initial state."""
    import mamba_selective_scan_s6_amd as S
    import oracle
    import torch

    cfg = W.DECODE_CONFIG
    prm = W.make_decode_params(cfg)
    ch = _sample_channels(cfg.nd, 4)
    state = to_dev(prm["state0"], dev)
    A, D = to_dev(prm["A"], dev), to_dev(prm["D"], dev)
    ref_state = prm["state0"][:, ch].astype(np.float64)
    A_s, D_s = prm["A"][ch].astype(np.float64), prm["D"][ch].astype(np.float64)
    for step in range(cfg.steps):
        si = W.make_decode_step(cfg.nb, cfg.nd, cfg.N, cfg.seed, step)
        t = _decode_inputs_dev(si, dev)
        out = decode_step(state, t, A, D, t["z"], check_bf16=step % 64 == 0)
        f = {k: W.bf16_bits_to_f64(v) for k, v in si.items()}
        ref_out, ref_state = oracle.state_update(ref_state, f["x"][:, ch], f["delta"][:, ch], A_s, f["B"], f["C"],
                                                 D_s, f["z"][:, ch])
        if step % 32 == 0 or step == cfg.steps - 1:
            torch.cuda.synchronize()
            assert_close(from_dev(out)[:, ch], ref_out, W.BF16, "decode step %d out" % step)
    torch.cuda.synchronize()
    assert_close(from_dev(state)[:, ch], ref_state, W.BF16, "decode final state")


@pytest.mark.parametrize("io", [W.F32, W.BF16])
def test_decode_steps_reproduce_scan(dev, io):
    """Iterating the decode update over a sequence from a zero state gives the scan's outputs and
    final state (softplus on, no bias); both are checked against the oracle's scan."""
    import mamba_selective_scan_s6_amd as S
    import torch

    nb, nd, L, N = 2, 96, 24, 16
    inp = W.make_scan_inputs(nb, nd, L, N, io, seed=31)
    ref_out, ref_st = run_oracle(inp, drop=("delta_bias",))
    state = torch.zeros((nb, nd, N), dtype=torch.float32, device=dev)
    A, D = to_dev(inp["A"], dev), to_dev(inp["D"], dev)
    outs = []
    for t in range(L):
        sl = {k: np.ascontiguousarray(inp[k][:, :, t]) for k in ("u", "delta", "z")}
        bc = {k: np.ascontiguousarray(inp[k][:, t, :]) for k in ("B", "C")}
        td = {"x": to_dev(sl["u"], dev), "delta": to_dev(sl["delta"], dev), "B": to_dev(bc["B"], dev),
              "C": to_dev(bc["C"], dev)}
        o = decode_step(state, td, A, D, to_dev(sl["z"], dev), check_bf16=io == W.BF16 and t % 8 == 0)
        outs.append(from_dev(o))
    got = np.stack(outs, axis=-1)
    assert_close(got, ref_out, io, "decode-as-scan out")
    assert_close(from_dev(state), ref_st, io, "decode-as-scan state")
    out_scan, st_scan = run_scan(inp, dev, drop=("delta_bias",), out_f32=True)
    assert_close(out_scan, ref_out, io, "scan out")


@pytest.mark.parametrize("nb,nd,N,io,drop", [(5, 100, 16, W.F32, ()),         # batch not a multiple of 4
                                              (3, 70, 5, W.BF16, ()),          # ragged channels, N < 16
                                              (6, 64, 16, W.BF16, ("D", "z")),  # no skip, no gate
                                              (1, 1, 1, W.F32, ())])
def test_decode_edge_shapes(dev, nb, nd, N, io, drop):
    """Three decode steps from a random state on ragged shapes, against the oracle's update."""
    import mamba_selective_scan_s6_amd as S
    import oracle
    import torch

    L = 3
    inp = W.make_scan_inputs(nb, nd, L, N, io, seed=nb * 100 + nd + N)
    rng = np.random.default_rng(7)
    st0 = (0.1 * rng.standard_normal((nb, nd, N))).astype(np.float32)
    state = to_dev(st0, dev)
    ref_state = st0.astype(np.float64)
    f = W.inputs_f64(inp)
    A = to_dev(inp["A"], dev)
    D = None if "D" in drop else to_dev(inp["D"], dev)
    for t in range(L):
        sl = {k: np.ascontiguousarray(inp[k][:, :, t]) for k in ("u", "delta", "z")}
        bc = {k: np.ascontiguousarray(inp[k][:, t, :]) for k in ("B", "C")}
        z = None if "z" in drop else to_dev(sl["z"], dev)
        td = {"x": to_dev(sl["u"], dev), "delta": to_dev(sl["delta"], dev), "B": to_dev(bc["B"], dev),
              "C": to_dev(bc["C"], dev)}
        out = decode_step(state, td, A, D, z, check_bf16=io == W.BF16)
        ref_out, ref_state = oracle.state_update(
            ref_state, f["u"][:, :, t], f["delta"][:, :, t], f["A"], f["B"][:, t, :], f["C"][:, t, :],
            None if "D" in drop else f["D"], None if "z" in drop else f["z"][:, :, t])
        torch.cuda.synchronize()
        assert_close(from_dev(out), ref_out, io, "decode step %d out" % t)
    assert_close(from_dev(state), ref_state, io, "decode final state")


# ---------------------------------------------------------------- sequence lengths and streams
def test_long_single_group_chain(dev):
    """One channel group, 131109 tokens: 2049 segments carried through one look-back chain; the
    oracle follows three channels (rows are independent)."""
    inp = W.make_scan_inputs(1, 64, 131109, 16, W.F32, seed=90)
    check_scan(inp, dev, channels=[0, 17, 63], what="1x64x131109")


@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 31, 63, 64, 65, 127, 128, 129])
def test_short_sequences(dev, L):
    """Lengths around the 16-token wave block and the 64-token segment."""
    inp = W.make_scan_inputs(2, 70, L, 16, W.BF16, seed=900 + L)
    check_scan(inp, dev, what="2x70x%d" % L)


def test_two_streams_concurrently(dev):
    """Two scans in flight at once on two streams (each stream has its own workspace), then the same
    problem on both streams; every result matches the oracle."""
    import mamba_selective_scan_s6_amd as S
    import torch

    probs = [W.make_scan_inputs(2, 200, 3000, 16, W.BF16, seed=91), W.make_scan_inputs(1, 130, 5000, 8, W.F32, seed=92)]
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    for rounds in range(2):
        pairs = [(probs[0], probs[1]), (probs[0], probs[0])][rounds]
        inputs = [{k: to_dev(inp.get(k), dev) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
                  for inp in pairs]
        torch.cuda.synchronize()  # every input resident, so that the two launches overlap
        results = []
        for inp, t, st in zip(pairs, inputs, streams):
            with torch.cuda.stream(st):
                results.append((inp, t, S.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                                        t["delta_bias"], out_f32=True)))
        for (inp, _, (out, last)), st in zip(results, streams):
            with torch.cuda.stream(st):
                S.stream_check()
            ref_out, ref_st = run_oracle(inp)
            assert_close(from_dev(out), ref_out, inp["io"], "stream out")
            assert_close(from_dev(last), ref_st, inp["io"], "stream last_state")


# ---------------------------------------------------------------- exact zero-order-hold input gain
@pytest.mark.parametrize("nb,nd,L,N,io", [(2, 100, 77, 16, W.F32), (3, 130, 300, 16, W.BF16), (1, 65, 513, 5, W.F32),
                                          (2, 70, 50, 3, W.BF16)])
def test_zoh_small_shapes(dev, nb, nd, L, N, io):
    inp = W.make_scan_inputs(nb, nd, L, N, io, seed=500 + nd + L + N)
    check_scan(inp, dev, zoh=True, what="zoh %dx%dx%d N%d %s" % (nb, nd, L, N, io))


@pytest.mark.parametrize("cfg_id", ["mamba130m", "mamba2p8b"])
def test_zoh_full_size_sampled(dev, cfg_id):
    cfg = W.SCAN_CONFIGS[cfg_id]
    inp = W.make_config_inputs(cfg)
    check_scan(inp, dev, channels=_sample_channels(cfg.nd, 50 + cfg.seed), zoh=True, what="zoh " + cfg.name)


@pytest.mark.parametrize("io", [W.F32, W.BF16])
def test_zoh_gain_branches(dev, io):
    """Steps from 1e-6 to 8 against A from 0 to -16: Delta A crosses the series / (abar - 1)/A switch at
    |Delta A| = 1/8 many times, and A = 0 takes the Delta limit."""
    nb, nd, L, N = 1, 64, 200, 16
    inp = W.make_scan_inputs(nb, nd, L, N, io, seed=77)
    rng = np.random.default_rng(78)
    steps = np.exp(rng.uniform(np.log(1e-6), np.log(8.0), size=(nb, nd, L)))
    inp["delta"] = W.to_io(steps, io)
    A = inp["A"].copy()
    A[::4, 0] = 0.0   # A = 0: the gain is Delta
    A[1::4, 5] = -1e-3
    inp["A"] = A
    inp["delta_bias"] = np.zeros(nd, np.float32)
    check_scan(inp, dev, softplus=False, zoh=True, what="zoh gain branches %s" % io)


@pytest.mark.parametrize("io", [W.F32, W.BF16])
def test_zoh_decode_steps_reproduce_scan(dev, io):
    import mamba_selective_scan_s6_amd as S
    import torch

    nb, nd, L, N = 5, 100, 20, 16
    inp = W.make_scan_inputs(nb, nd, L, N, io, seed=79)
    ref_out, ref_st = run_oracle(inp, drop=("delta_bias",), zoh=True)
    state = torch.zeros((nb, nd, N), dtype=torch.float32, device=dev)
    A, D = to_dev(inp["A"], dev), to_dev(inp["D"], dev)
    outs = []
    for t in range(L):
        sl = {k: np.ascontiguousarray(inp[k][:, :, t]) for k in ("u", "delta", "z")}
        bc = {k: np.ascontiguousarray(inp[k][:, t, :]) for k in ("B", "C")}
        td = {"x": to_dev(sl["u"], dev), "delta": to_dev(sl["delta"], dev), "B": to_dev(bc["B"], dev),
              "C": to_dev(bc["C"], dev)}
        o = decode_step(state, td, A, D, to_dev(sl["z"], dev), check_bf16=io == W.BF16 and t % 8 == 0, zoh=True)
        outs.append(from_dev(o))
    assert_close(np.stack(outs, axis=-1), ref_out, io, "zoh decode-as-scan out")
    assert_close(from_dev(state), ref_st, io, "zoh decode-as-scan state")


# ---------------------------------------------------------------- causal convolution + SiLU
def _conv_inputs(nb, nd, L, K, io, seed, with_bias=True):
    rng = np.random.default_rng(seed)
    x = W.to_io(rng.standard_normal((nb, nd, L)), io)
    w = (0.5 * rng.standard_normal((nd, K))).astype(np.float32)
    b = (0.1 * rng.standard_normal(nd)).astype(np.float32) if with_bias else None
    return x, w, b


@pytest.mark.parametrize("nb,nd,L,K,io,silu,bias", [(2, 100, 77, 4, W.F32, True, True), (3, 130, 300, 4, W.BF16, True, True),
                                                    (1, 64, 2048, 4, W.BF16, False, True), (2, 33, 5, 4, W.F32, True, False),
                                                    (1, 17, 1, 4, W.BF16, True, True), (2, 40, 64, 1, W.F32, True, True),
                                                    (2, 40, 65, 2, W.BF16, True, True), (1, 50, 99, 3, W.F32, False, False),
                                                    (2, 40, 120, 8, W.BF16, True, True), (1, 1536, 2048, 4, W.F32, True, True),
                                                    (2, 2048, 2050, 4, W.BF16, True, True),   # 16 tokens per lane, ragged
                                                    (4, 1024, 2048, 4, W.F32, True, True),    # 16 tokens per lane
                                                    # 16 tokens per lane at the extreme widths (halo of 7, none)
                                                    (1, 4096, 2048, 8, W.BF16, False, False),
                                                    (2, 1024, 4096, 1, W.BF16, True, True),
                                                    # short rows at the edge of the vector path (its halo vector
                                                    # of a row's first chunk covers elements 0..7)
                                                    (2, 70, 4, 4, W.F32, True, True), (2, 70, 8, 8, W.F32, True, True),
                                                    (1, 65, 12, 8, W.F32, True, True), (1, 64, 24, 8, W.BF16, True, True),
                                                    # widths 2 and 3 on shapes large enough for 16 tokens per lane
                                                    # (the kernels with the width fixed at compile time)
                                                    (2, 2048, 2048, 3, W.BF16, True, True), (4, 1024, 2048, 2, W.F32, False, True)])
def test_causal_conv1d(dev, nb, nd, L, K, io, silu, bias):
    import mamba_selective_scan_s6_amd as S
    import oracle

    x, w, b = _conv_inputs(nb, nd, L, K, io, seed=nb * 7 + nd + L + K, with_bias=bias)
    got = S.causal_conv1d(to_dev(x, dev), to_dev(w, dev), to_dev(b, dev), silu=silu)
    ref = oracle.causal_conv1d(W.io_to_f64(x, io), w, b, silu_flag=silu)
    check = assert_close if io == W.F32 else assert_close_before_cast
    check(from_dev(got), ref, io, "conv %dx%dx%d K%d" % (nb, nd, L, K))


@pytest.mark.parametrize("io,K", [(W.F32, 4), (W.BF16, 4), (W.BF16, 3)])
def test_conv_window_steps_reproduce_sequence(dev, io, K):
    """Decode steps from a zero window give the sequence convolution token by token (both against
    the oracle), and the window ends holding the last K inputs."""
    import mamba_selective_scan_s6_amd as S
    import oracle
    import torch

    nb, nd, L = 5, 70, 12
    x, w, b = _conv_inputs(nb, nd, L, K, io, seed=60 + K)
    ref = oracle.causal_conv1d(W.io_to_f64(x, io), w, b)
    win = torch.zeros((nb, nd, K), dtype=torch.float32, device=dev)
    wd, bd = to_dev(w, dev), to_dev(b, dev)
    for t in range(L):
        o = S.conv_window_update(win, to_dev(np.ascontiguousarray(x[:, :, t]), dev), wd, bd)
        check = assert_close if io == W.F32 else assert_close_before_cast
        check(from_dev(o), ref[:, :, t], io, "window step %d" % t)
    np.testing.assert_array_equal(from_dev(win), W.io_to_f64(x, io)[:, :, L - K:])


# ---------------------------------------------------------------- workspace, launch tags, checks
def test_repeated_launches_and_workspace_growth(dev):
    """Launches reuse the stream's workspace under fresh launch tags, across shapes; a larger problem
    gets a larger workspace. Every result matches the oracle and no cross-workgroup wait timed out."""
    import mamba_selective_scan_s6_amd as S

    small = W.make_scan_inputs(1, 64, 96, 16, W.F32, seed=51)
    big = W.make_scan_inputs(2, 192, 700, 16, W.BF16, seed=52)
    for inp in (small, small, big, small, big):
        check_scan(inp, dev, what="repeat")
    S.stream_check()


def test_timed_out_wait_is_reported_then_cleared(dev):
    """With the look-back allowed a single poll, segments that find a predecessor unpublished give up
    and record a timeout; the kernel still finishes, stream_check raises SSM_ERR_DEVICE_WAIT once,
    and with the default limit the next launch is correct again."""
    import mamba_selective_scan_s6_amd as S

    inp = W.make_scan_inputs(1, 64, 131072, 16, W.BF16, seed=95)  # 2048 segments of one group in flight
    prev = S.set_wait_limit(1)
    try:
        t = {k: to_dev(inp.get(k), dev) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
        S.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
        with pytest.raises(S.SSMError) as err:
            S.stream_check()
        assert err.value.status == 6  # SSM_ERR_DEVICE_WAIT
    finally:
        S.set_wait_limit(prev)
    S.stream_check()  # cleared by the previous check
    check_scan(inp, dev, channels=[0, 31, 63], what="after a reported timeout")


def test_scan_after_releasing_workspaces(dev):
    import mamba_selective_scan_s6_amd as S

    inp = W.make_scan_inputs(2, 130, 700, 16, W.F32, seed=96)
    check_scan(inp, dev, what="before release")
    S.release_workspaces()
    check_scan(inp, dev, what="after release")


def test_stream_check_reports_clean(dev):
    import mamba_selective_scan_s6_amd as S

    inp = W.make_config_inputs(W.SCAN_CONFIGS["mamba130m"])
    run_scan(inp, dev)
    S.stream_check()  # raises SSMError if any wait timed out
