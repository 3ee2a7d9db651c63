"""GPU tests of the contracts around the kernels, each against the fp64 oracle.

* Resume: a scan over tokens [0, L1) whose last_state seeds decode steps over [L1, L) gives the outputs
  and final state of one scan over [0, L) ("Beyond attention with Mamba, state space models and
  hybrids", section 7: generation carries a state of fixed size from the prompt's scan).
* Graph capture: a scan, backward or SSD scan captured in a HIP graph, with a caller-owned workspace,
  stays correct on every replay while the inputs change between replays (the scan kernels keep their
  launch tag in the workspace, not in the captured arguments; the SSD's workspace holds nothing between
  calls). Every replay is compared bit for bit with an eager call on the same inputs, with eager work
  and synchronisations between replays, and the scans' replays with the oracle at the parity tolerance."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import TOL, assert_close, from_dev, to_dev

pytestmark = pytest.mark.gpu

FIELDS = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import mamba_selective_scan_s6_amd as S

    S.load_library()
    return torch.device("cuda:0")


def oracle_scan(inp, zoh=False, drop=()):
    import oracle

    f = W.inputs_f64(inp)
    for k in drop:
        f[k] = None
    return oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"], f["delta_bias"], zoh=zoh)


@pytest.mark.parametrize("io,zoh,L,L1", [(W.F32, False, 200, 130), (W.BF16, False, 200, 64), (W.BF16, True, 150, 97),
                                          (W.F32, True, 70, 1)])
def test_prefill_then_decode_resumes_the_scan(dev, io, zoh, L, L1):
    import mamba_selective_scan_s6_amd as S
    import torch

    nb, nd, N = 2, 130, 16
    inp = W.make_scan_inputs(nb, nd, L, N, io, seed=700 + L + L1)
    ref_out, ref_state = oracle_scan(inp, zoh=zoh, drop=("delta_bias",))  # decode steps take no bias
    pre = {k: inp[k] for k in ("A", "D")}
    for k in ("u", "delta", "z"):
        pre[k] = np.ascontiguousarray(inp[k][:, :, :L1])
    for k in ("B", "C"):
        pre[k] = np.ascontiguousarray(inp[k][:, :L1, :])
    t = {k: to_dev(pre[k], dev) for k in pre}
    out, state = S.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], None, zoh=zoh,
                                out_f32=True)
    S.stream_check()
    assert_close(from_dev(out), ref_out[:, :, :L1], io, "prefill out")
    A, D = t["A"], t["D"]
    outs = []
    for step in range(L1, L):
        x = to_dev(np.ascontiguousarray(inp["u"][:, :, step]), dev)
        dl = to_dev(np.ascontiguousarray(inp["delta"][:, :, step]), dev)
        z = to_dev(np.ascontiguousarray(inp["z"][:, :, step]), dev)
        Bt = to_dev(np.ascontiguousarray(inp["B"][:, step, :]), dev)
        Ct = to_dev(np.ascontiguousarray(inp["C"][:, step, :]), dev)
        outs.append(S.ssm_state_update(state, x, dl, A, Bt, Ct, D, z, zoh=zoh, out_f32=True))
    torch.cuda.synchronize()
    got = np.stack([from_dev(o) for o in outs], axis=-1)
    assert_close(got, ref_out[:, :, L1:], io, "decode continuation out")
    assert_close(from_dev(state), ref_state, io, "final state after prefill + decode")


def _capture(torch, fn):
    """Warm up `fn` on a side stream, then capture it; returns (graph, outputs of the captured call)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    torch.cuda.synchronize()
    return g, res


@pytest.mark.parametrize("io", [W.BF16, W.F32])
def test_scan_in_a_graph_replays_correctly_with_new_inputs(dev, io):
    import mamba_selective_scan_s6_amd as S
    import torch

    nb, nd, L, N = 2, 200, 700, 16   # 4 channel groups x 11 segments: carries cross workgroups
    first = W.make_scan_inputs(nb, nd, L, N, io, seed=800)
    static = {k: to_dev(first[k], dev) for k in FIELDS}
    ws = torch.zeros(S.scan_workspace_size(nb, nd, L), dtype=torch.uint8, device=dev)

    def call():
        return S.ssm_scan_fwd(*(static[k] for k in FIELDS), workspace=ws, out_f32=True)

    g, (out, state) = _capture(torch, call)
    for rep in range(4):
        inp = W.make_scan_inputs(nb, nd, L, N, io, seed=801 + rep)
        for k in FIELDS:
            static[k].copy_(to_dev(inp[k], dev))
        g.replay()
        torch.cuda.synchronize()
        got_out, got_state = out.clone(), state.clone()
        e_out, e_state = S.ssm_scan_fwd(*(static[k] for k in FIELDS), out_f32=True)  # eager, its own workspace
        S.stream_check()
        S.workspace_check(ws)
        assert torch.equal(got_out, e_out), "replay %d: out differs from the eager call" % rep
        assert torch.equal(got_state, e_state), "replay %d: last_state differs from the eager call" % rep
        if rep in (0, 3):
            ref_out, ref_state = oracle_scan(inp)
            assert_close(from_dev(got_out), ref_out, io, "replay %d out" % rep)
            assert_close(from_dev(got_state), ref_state, io, "replay %d last_state" % rep)


def test_backward_in_a_graph_replays_correctly_with_new_inputs(dev):
    import mamba_selective_scan_s6_amd as S
    import torch

    nb, nd, L, N, io = 1, 130, 300, 16, W.F32
    first = W.make_scan_inputs(nb, nd, L, N, io, seed=900)
    static = {k: to_dev(first[k], dev) for k in FIELDS}
    static["dout"] = to_dev(W.to_io(np.random.default_rng(900).standard_normal(first["u"].shape), io), dev)
    ws = torch.zeros(S.scan_bwd_workspace_size(nb, nd, L), dtype=torch.uint8, device=dev)

    def call():
        return S.ssm_scan_bwd(*(static[k] for k in FIELDS), dout=static["dout"], workspace=ws)

    g, grads = _capture(torch, call)
    for rep in range(3):
        inp = W.make_scan_inputs(nb, nd, L, N, io, seed=901 + rep)
        dout = W.to_io(np.random.default_rng(901 + rep).standard_normal(inp["u"].shape), io)
        for k in FIELDS:
            static[k].copy_(to_dev(inp[k], dev))
        static["dout"].copy_(to_dev(dout, dev))
        g.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in grads.items() if v is not None}
        eager = S.ssm_scan_bwd(*(static[k] for k in FIELDS), dout=static["dout"])
        S.stream_check()
        S.workspace_check(ws)
        for k, v in got.items():
            assert torch.equal(v, eager[k]), "replay %d: %s differs from the eager call" % (rep, k)
        if rep == 2:
            import oracle

            f = W.inputs_f64(inp)
            ref = oracle.scan_bwd(*(f[k] for k in FIELDS), dout=W.io_to_f64(dout, io), softplus_flag=True)
            for k in ("du", "ddelta", "dz"):
                assert_close(from_dev(got[k]), ref[k], io, "replay %d %s" % (rep, k))
            rtol = TOL[io][0]
            for k in ("dA", "dB", "dC", "dD", "ddelta_bias"):
                r = np.asarray(ref[k])
                err = np.abs(from_dev(got[k]) - r)
                assert np.all(err <= rtol * np.abs(r) + rtol * np.max(np.abs(r))), k


def test_ssd_in_a_graph_replays_correctly_with_new_inputs(dev):
    """The SSD scan's three kernels (segment states, carries, outputs) captured in a HIP graph with a
    caller-owned workspace: every replay equals an eager call on the same inputs, bit for bit."""
    import mamba_selective_scan_s6_amd as S
    import torch

    nb, L, H, P, N, G, io = 1, 700, 3, 32, 64, 1, W.BF16
    code = S.BF16
    need = S.ssd_workspace_size(nb, L, H, P, N, code)
    assert need > 0, "the shape must take the split form"
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    keys = ("x", "a", "b", "c")
    static = {k: to_dev(v, dev) for k, v in W.make_ssd_inputs(nb, L, H, P, N, G, io, seed=950).items() if k in keys}

    def call():
        return S.ssd_scan(*(static[k] for k in keys), workspace=ws, out_f32=True)

    g, (y, fs) = _capture(torch, call)
    for rep in range(3):
        inp = W.make_ssd_inputs(nb, L, H, P, N, G, io, seed=951 + rep)
        for k in keys:
            static[k].copy_(to_dev(inp[k], dev))
        g.replay()
        torch.cuda.synchronize()
        got_y, got_f = y.clone(), fs.clone()
        e_y, e_f = S.ssd_scan(*(static[k] for k in keys), out_f32=True)  # eager, the binding's own workspace
        torch.cuda.synchronize()
        assert torch.equal(got_y, e_y), "replay %d: y differs from the eager call" % rep
        assert torch.equal(got_f, e_f), "replay %d: final state differs from the eager call" % rep

