"""Pins for the fp64 oracle: values the pages print, closed forms, invariants, and an
independent log-depth scan. None of these re-types the oracle's own loop; each checks it
against something the pages or the mathematics fix, chosen so that a dropped term, a wrong
sign or index, or a transposed operand in the oracle fails at least one of them."""
import math

import numpy as np
import pytest

from conftest import golden
from workloads import softplus_inverse

pytestmark = pytest.mark.filterwarnings("ignore")


def scan1(oracle, u, dt, a, b, c, D=None, z=None, bias=None, softplus=False, zoh=False):
    """Single channel, single state, scalar or per-token coefficients."""
    u = np.asarray(u, dtype=np.float64)
    L = u.size
    dt = np.broadcast_to(np.asarray(dt, dtype=np.float64), (L,))
    b = np.broadcast_to(np.asarray(b, dtype=np.float64), (L,))
    c = np.broadcast_to(np.asarray(c, dtype=np.float64), (L,))
    out, st = oracle.scan_fwd(u.reshape(1, 1, L), dt.reshape(1, 1, L), np.array([[a]], dtype=np.float64),
                              b.reshape(1, L, 1), c.reshape(1, L, 1),
                              None if D is None else np.array([D], dtype=np.float64),
                              None if z is None else np.asarray(z, dtype=np.float64).reshape(1, 1, L),
                              None if bias is None else np.array([bias], dtype=np.float64),
                              softplus_flag=softplus, zoh=zoh)
    return out.reshape(L), st.reshape(-1)


def hillis_steele(a, b):
    """Inclusive scan of h_t = a_t h_{t-1} + b_t by log-depth rounds: in round k every position
    composes with the one 2^k to its left (identity a = 1, b = 0 beyond the start)."""
    a = np.array(a, dtype=np.float64)
    h = np.array(b, dtype=np.float64)
    shift, rounds = 1, 0
    while shift < a.size:
        a_left = np.concatenate([np.ones(shift), a[:-shift]])
        h_left = np.concatenate([np.zeros(shift), h[:-shift]])
        h = a * h_left + h
        a = a * a_left
        shift *= 2
        rounds += 1
    return h, rounds


# ------------------------------------------------------------------ values printed on the pages
def test_p5_toy_recurrence(oracle_mod):
    g = golden("p5_toy_recurrence.json")
    # Delta = 1 with softplus off: Abar = exp(a) -> a = ln 0.8; Euler Bbar = Delta * B = 0.2.
    out, st = scan1(oracle_mod, g["inputs"], 1.0, math.log(g["Abar"]), g["Bbar"], 1.0)
    assert np.round(out, g["decimals"]).tolist() == g["states"]
    assert out[3] == pytest.approx(2.512, abs=1e-12)
    assert st[0] == pytest.approx(out[-1], abs=0)


def test_m19_impulse_response(oracle_mod):
    g = golden("m19_impulse_response.json")
    out, _ = scan1(oracle_mod, g["x"], 1.0, math.log(g["Abar"]), g["Bbar"], g["C"])
    assert np.round(out, g["decimals"]).tolist() == g["y"]


def test_m19_parallel_scan_example(oracle_mod):
    g = golden("m19_parallel_scan.json")
    a, b = np.array(g["a"]), np.array(g["b"])
    # Through the real API: A = -1 and Delta_t = -ln a_t give Abar_t = a_t; B_t = b_t / Delta_t with
    # u = 1 gives the write Delta_t B_t u_t = b_t.
    dt = -np.log(a)
    out, _ = scan1(oracle_mod, np.ones(5), dt, -1.0, b / dt, 1.0)
    assert np.round(out, g["decimals"]).tolist() == g["h"]
    hs, rounds = hillis_steele(a, b)
    np.testing.assert_allclose(out, hs, rtol=1e-13, atol=1e-15)
    assert rounds == 3


def test_m19_discretize_zoh(oracle_mod):
    g = golden("m19_discretize.json")
    A = np.array(g["A"])
    N = A.size
    u = np.array([[[1.0, 0.0]]])
    dt = np.full((1, 1, 2), g["delta"])
    B = np.tile(np.array(g["B"]), (1, 2, 1))
    C = np.zeros((1, 2, N))
    _, st1 = oracle_mod.scan_fwd(u[:, :, :1], dt[:, :, :1], A.reshape(1, N), B[:, :1], C[:, :1],
                                 softplus_flag=False, zoh=True)
    _, st2 = oracle_mod.scan_fwd(u, dt, A.reshape(1, N), B, C, softplus_flag=False, zoh=True)
    bbar = st1.reshape(N)        # one step from zero with u = 1: h = Bbar
    abar = st2.reshape(N) / bbar  # a second step with u = 0: h = Abar Bbar
    assert np.round(abar, g["decimals"]).tolist() == g["Abar"]
    assert np.round(bbar, g["decimals"]).tolist() == g["Bbar"]
    # Abar is in (0, 1) for a < 0, and Euler mode keeps the same decay.
    _, st2e = oracle_mod.scan_fwd(u, dt, A.reshape(1, N), B, C, softplus_flag=False, zoh=False)
    np.testing.assert_allclose(st2e.reshape(N) / g["delta"], abar, rtol=1e-14)


def test_p4_zoh_over_euler_ratio(oracle_mod):
    g = golden("p4_zoh_euler_ratio.json")
    got = []
    for p in g["abs_delta_a"]:
        _, zoh = scan1(oracle_mod, [1.0], p, -1.0, 1.0, 0.0, zoh=True)
        _, eul = scan1(oracle_mod, [1.0], p, -1.0, 1.0, 0.0, zoh=False)
        got.append(round(float(zoh[0] / eul[0]), g["decimals"]))
    assert got == g["ratio"]


def test_p5_retention(oracle_mod):
    g = golden("p5_retention.json")
    for case in g["cases"]:
        # Decode step from state 1 with no input: the state keeps exp(Delta a). The decode step
        # always applies softplus, so feed softplus^-1(Delta).
        raw = float(softplus_inverse(case["delta"]))
        _, st = oracle_mod.state_update(np.ones((1, 1, 1)), np.zeros((1, 1)), np.array([[raw]]),
                                        np.array([[g["A"]]]), np.zeros((1, 1)), np.zeros((1, 1)))
        assert round(100 * float(st.reshape(-1)[0])) == case["kept_percent"]
        # The scan path gives the same decay between two tokens.
        out, _ = scan1(oracle_mod, [1.0, 0.0], case["delta"], g["A"], 1.0, 1.0)
        assert round(100 * out[1] / out[0]) == case["kept_percent"]
    assert math.exp(-0.1) == pytest.approx(0.905, abs=5e-4)
    assert math.exp(-2.0) == pytest.approx(0.135, abs=5e-4)


def test_p5_selectivity_toy(oracle_mod):
    g = golden("p5_selectivity.json")
    sel, fix = g["selective"], g["fixed"]
    u = np.zeros(1 + sel["fillers"])
    u[0] = 1.0
    dt = np.full(u.size, sel["filler_delta"])
    dt[0] = sel["key_delta"]
    _, st = scan1(oracle_mod, u, dt, g["A"], g["B"], 0.0, zoh=True)
    assert round(100 * st[0], sel["decimals"]) == sel["survives_percent"]
    assert st[0] == pytest.approx((1 - math.exp(-5)) * math.exp(-0.09), rel=1e-13)
    _, st = scan1(oracle_mod, u, fix["delta"], g["A"], g["B"], 0.0, zoh=True)
    assert round(100 * st[0], fix["decimals"]) == fix["survives_percent"]
    # Under the Euler gain the same toy would not give the printed figures.
    _, st_e = scan1(oracle_mod, u, dt, g["A"], g["B"], 0.0, zoh=False)
    assert round(100 * st_e[0]) != sel["survives_percent"]


def test_m19_kernel_taps_and_convolution_face(oracle_mod):
    torch = pytest.importorskip("torch")
    g = golden("m19_kernel_taps.json")
    torch.manual_seed(0)
    abar = (torch.rand(4) * 0.9 + 0.05).double().numpy()
    bbar = torch.randn(4).double().numpy()
    c = torch.randn(4).double().numpy()
    x = torch.randn(16).double().numpy()

    def run(u):
        L = u.size
        out, _ = oracle_mod.scan_fwd(u.reshape(1, 1, L), np.ones((1, 1, L)), np.log(abar).reshape(1, 4),
                                     np.tile(bbar, (1, L, 1)), np.tile(c, (1, L, 1)), softplus_flag=False)
        return out.reshape(L)

    impulse = np.zeros(4)
    impulse[0] = 1.0
    taps = run(impulse)
    assert np.round(taps, g["decimals"]).tolist() == g["taps"]
    # Convolution face: y_t = sum_i K_i x_{t-i}, K_i = sum_n C_n Abar_n^i Bbar_n (time-invariant case).
    K = np.array([np.sum(c * abar ** i * bbar) for i in range(16)])
    y_conv = np.array([sum(K[i] * x[t - i] for i in range(t + 1)) for t in range(16)])
    y_rec = run(x)
    np.testing.assert_allclose(y_rec, y_conv, rtol=1e-12, atol=1e-14)
    assert np.max(np.abs(y_rec - y_conv)) < g["rec_vs_conv_atol"]


def test_scan_rounds_and_log_depth_scan(oracle_mod):
    g = golden("scan_rounds.json")
    rng = np.random.default_rng(7)
    for case in g["cases"]:
        L = case["length"]
        a = rng.uniform(0.05, 0.95, L)
        b = rng.standard_normal(L)
        dt = -np.log(a)
        out, st = scan1(oracle_mod, np.ones(L), dt, -1.0, b / dt, 1.0)
        hs, rounds = hillis_steele(a, b)
        assert rounds == case["rounds"] == math.ceil(math.log2(L))
        np.testing.assert_allclose(out, hs, rtol=1e-12, atol=1e-13)
        assert st[0] == out[-1]
        if "sequential_steps" in case:
            assert case["sequential_steps"] == L - 1


# ------------------------------------------------------------------ closed forms and special cases
def test_softplus_values_and_inverse(oracle_mod):
    sp = oracle_mod.softplus
    assert sp(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert sp(40.0) == pytest.approx(40.0, rel=1e-15)           # log(1 + e^r) -> r
    assert sp(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-14, abs=0)  # -> e^r, relative accuracy kept
    assert sp(1.0) == pytest.approx(math.log(1.0 + math.e), rel=1e-15)
    assert sp(-1.0) == pytest.approx(math.log(1.0 + 1.0 / math.e), rel=1e-15)
    # The dt initialisation inverts softplus ("Beyond attention with Mamba ...", section 11).
    dts = np.exp(np.linspace(math.log(1e-3), math.log(1e-1), 41))
    for dt in dts:
        assert sp(float(softplus_inverse(dt))) == pytest.approx(dt, rel=1e-12, abs=0)


def test_gate_closed_forms(oracle_mod):
    # B = 0 keeps the state at zero, so out = D u SiLU(z); sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4.
    z = np.array([math.log(3.0), -math.log(3.0), 0.0, 30.0])
    out, _ = scan1(oracle_mod, np.ones(4), 0.3, -1.0, 0.0, 1.0, D=1.0, z=z)
    np.testing.assert_allclose(out, [0.75 * math.log(3.0), -0.25 * math.log(3.0), 0.0, 30.0], rtol=1e-13, atol=1e-30)
    assert oracle_mod.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)


def test_skip_term(oracle_mod):
    out, st = scan1(oracle_mod, [2.0, -1.0, 4.0], 0.7, -2.0, 0.0, 1.0, D=2.5)
    np.testing.assert_array_equal(out, [5.0, -2.5, 10.0])
    assert st[0] == 0.0
    out_nod, _ = scan1(oracle_mod, [2.0, -1.0, 4.0], 0.7, -2.0, 0.0, 1.0)
    np.testing.assert_array_equal(out_nod, [0.0, 0.0, 0.0])


def test_bias_inside_softplus(oracle_mod):
    # Delta = softplus(raw + bias): raw = 0 and bias = softplus^-1(0.25) give Delta = 0.25, so with
    # A = 0 (Abar = 1) and B = 1 the state sums 0.25 * u.
    bias = float(softplus_inverse(0.25))
    out, st = scan1(oracle_mod, [1.0, 1.0, 2.0], 0.0, 0.0, 1.0, 1.0, bias=bias, softplus=True)
    np.testing.assert_allclose(out, [0.25, 0.5, 1.0], rtol=1e-13)
    # softplus off: Delta = raw + bias exactly.
    out, _ = scan1(oracle_mod, [1.0, 1.0], 0.5, 0.0, 1.0, 1.0, bias=0.25, softplus=False)
    np.testing.assert_allclose(out, [0.75, 1.5], rtol=1e-15)


def test_zero_step_and_zero_a_limits(oracle_mod):
    # Delta = 0: Abar = 1 and nothing is written; out = D u SiLU(z) only.
    out, st = scan1(oracle_mod, [3.0, -2.0], 0.0, -5.0, 1.0, 1.0, D=1.0)
    np.testing.assert_array_equal(out, [3.0, -2.0])
    assert st[0] == 0.0
    # a = 0 under the exact rule falls back to the Euler limit Delta B ("Module 19", The Math).
    out_z, _ = scan1(oracle_mod, [1.0, 1.0, 1.0], 0.2, 0.0, 2.0, 1.0, zoh=True)
    out_e, _ = scan1(oracle_mod, [1.0, 1.0, 1.0], 0.2, 0.0, 2.0, 1.0, zoh=False)
    np.testing.assert_allclose(out_z, [0.4, 0.8, 1.2], rtol=1e-14)
    np.testing.assert_array_equal(out_z, out_e)
    # A large step with a < 0 resets the state: Abar -> 0.
    out, _ = scan1(oracle_mod, [5.0, 1.0], [0.1, 60.0], -1.0, 1.0, 1.0)
    assert out[1] == pytest.approx(60.0, rel=1e-12)


def test_exercise3_selective_copy_closed_form(oracle_mod):
    # "Module 19", Exercise 3: Delta high at one position, low elsewhere, B = C = 1, A = -1.
    rng = np.random.default_rng(3)
    u = rng.standard_normal(8)
    dt = np.full(8, 0.02)
    dt[2] = 1.5
    out, _ = scan1(oracle_mod, u, dt, -1.0, 1.0, 1.0)
    h = 0.0
    for t in range(8):
        h = math.exp(-dt[t]) * h + dt[t] * u[t]
        assert out[t] == pytest.approx(h, rel=1e-14, abs=1e-16)
    # After the key the output decays by exactly e^{-0.02} per step plus 0.02 u.
    for t in range(3, 8):
        assert out[t] == pytest.approx(math.exp(-0.02) * out[t - 1] + 0.02 * u[t], rel=1e-13)


# ------------------------------------------------------------------ invariants and structure
def _rand_case(rng, nb, nd, L, N):
    return dict(u=rng.standard_normal((nb, nd, L)), delta=0.5 * rng.standard_normal((nb, nd, L)),
                A=-rng.uniform(0.5, 4.0, (nd, N)), B=rng.standard_normal((nb, L, N)),
                C=rng.standard_normal((nb, L, N)), D=rng.uniform(0.5, 1.5, nd),
                z=rng.standard_normal((nb, nd, L)), delta_bias=rng.uniform(-4.0, -1.0, nd))


def test_rows_are_independent_and_indexed_right(oracle_mod):
    """Each (batch, channel) row of a multi-row run equals a one-row run fed that row's slices:
    B/C by batch, A/D/bias by channel, u/delta/z by both (catches swapped or transposed indices)."""
    rng = np.random.default_rng(11)
    nb, nd, L, N = 2, 3, 7, 5
    k = _rand_case(rng, nb, nd, L, N)
    out, st = oracle_mod.scan_fwd(**k, softplus_flag=True)
    for b in range(nb):
        for d in range(nd):
            o1, s1 = oracle_mod.scan_fwd(k["u"][b:b + 1, d:d + 1], k["delta"][b:b + 1, d:d + 1], k["A"][d:d + 1],
                                         k["B"][b:b + 1], k["C"][b:b + 1], k["D"][d:d + 1], k["z"][b:b + 1, d:d + 1],
                                         k["delta_bias"][d:d + 1], softplus_flag=True)
            np.testing.assert_array_equal(out[b, d], o1[0, 0])
            np.testing.assert_array_equal(st[b, d], s1[0, 0])


def test_readout_sums_independent_states(oracle_mod):
    """With no skip and no gate, out is the sum over states of single-state runs (state n uses
    column n of A, B, C); the state vector is the per-state states."""
    rng = np.random.default_rng(12)
    nb, nd, L, N = 1, 2, 9, 4
    k = _rand_case(rng, nb, nd, L, N)
    out, st = oracle_mod.scan_fwd(k["u"], k["delta"], k["A"], k["B"], k["C"], None, None, k["delta_bias"])
    acc = np.zeros_like(out)
    for n in range(N):
        o, s = oracle_mod.scan_fwd(k["u"], k["delta"], k["A"][:, n:n + 1], k["B"][:, :, n:n + 1],
                                   k["C"][:, :, n:n + 1], None, None, k["delta_bias"])
        acc += o
        np.testing.assert_allclose(st[:, :, n], s[:, :, 0], rtol=1e-15)
    np.testing.assert_allclose(out, acc, rtol=1e-12, atol=1e-14)


def test_linearity_in_u(oracle_mod):
    rng = np.random.default_rng(13)
    k = _rand_case(rng, 1, 3, 20, 4)
    u1, u2 = k["u"], rng.standard_normal(k["u"].shape)
    base = dict(delta=k["delta"], A=k["A"], B=k["B"], C=k["C"], D=k["D"], z=None, delta_bias=k["delta_bias"])
    o1, s1 = oracle_mod.scan_fwd(u1, **base)
    o2, s2 = oracle_mod.scan_fwd(u2, **base)
    o12, s12 = oracle_mod.scan_fwd(u1 + u2, **base)
    np.testing.assert_allclose(o12, o1 + o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s12, s1 + s2, rtol=1e-11, atol=1e-12)
    o3, _ = oracle_mod.scan_fwd(-2.5 * u1, **base)
    np.testing.assert_allclose(o3, -2.5 * o1, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("field", ["u", "delta", "z", "B", "C"])
def test_causality_bitwise(oracle_mod, field):
    rng = np.random.default_rng(14)
    nb, nd, L, N = 2, 3, 16, 4
    k = _rand_case(rng, nb, nd, L, N)
    out, _ = oracle_mod.scan_fwd(**k)
    t = 9
    k2 = {kk: (v.copy() if isinstance(v, np.ndarray) else v) for kk, v in k.items()}
    if field in ("B", "C"):
        k2[field][:, t, :] += 4.0
    else:
        k2[field][:, :, t] += 4.0
    out2, _ = oracle_mod.scan_fwd(**k2)
    np.testing.assert_array_equal(out[:, :, :t], out2[:, :, :t])
    assert np.all(out[:, :, t] != out2[:, :, t])


def test_decode_steps_equal_scan(oracle_mod):
    """L decode steps from a zero state give the scan's outputs and final state ("Beyond attention
    with Mamba ...", section 7: step by step against the whole sequence). The scan runs with
    softplus on and no bias, the decode step's fixed step rule."""
    rng = np.random.default_rng(15)
    nb, nd, L, N = 2, 3, 12, 4
    k = _rand_case(rng, nb, nd, L, N)
    out, st = oracle_mod.scan_fwd(k["u"], k["delta"], k["A"], k["B"], k["C"], k["D"], k["z"], None, softplus_flag=True)
    state = np.zeros((nb, nd, N))
    for t in range(L):
        o, state = oracle_mod.state_update(state, k["u"][:, :, t], k["delta"][:, :, t], k["A"], k["B"][:, t],
                                           k["C"][:, t], k["D"], k["z"][:, :, t])
        np.testing.assert_allclose(o, out[:, :, t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(state, st, rtol=1e-12, atol=1e-14)


def test_thread_count_does_not_change_bits(oracle_mod):
    rng = np.random.default_rng(16)
    k = _rand_case(rng, 2, 9, 33, 16)
    o1, s1 = oracle_mod.scan_fwd(**k, nthreads=1)
    o4, s4 = oracle_mod.scan_fwd(**k, nthreads=4)
    o7, s7 = oracle_mod.scan_fwd(**k, nthreads=7)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(o1, o7)
    np.testing.assert_array_equal(s1, s7)


def test_state_size_arithmetic():
    # "State space models vs attention ...": a layer 2,048 wide with expansion 2 and N = 16 holds
    # 128 KiB in 16-bit numbers, the quantity the decode state of one batch row occupies.
    assert 2048 * 2 * 16 * 2 == 128 * 1024


# ------------------------------------------------------------------ causal depthwise convolution
# "Module 19: State-Space Models (Mamba)", The Causal Convolution; "Beyond attention with Mamba,
# state space models and hybrids", section 4 (conv1d, left padding K-1, cropped) and section 7
# (mixer_step's window of the last inputs).
def _silu(v):
    return v / (1.0 + np.exp(-v))


def test_conv_first_token_sees_one_tap(oracle_mod):
    """At t = 0 the window has a single valid tap, the newest one; the rest is the zero left pad."""
    rng = np.random.default_rng(30)
    x = rng.standard_normal((2, 3, 9))
    w = rng.standard_normal((3, 4))
    b = rng.standard_normal(3)
    out = oracle_mod.causal_conv1d(x, w, b, silu_flag=False)
    np.testing.assert_allclose(out[:, :, 0], b + w[:, 3] * x[:, :, 0], rtol=1e-15, atol=1e-15)
    # t = 1: the two newest taps
    np.testing.assert_allclose(out[:, :, 1], b + w[:, 2] * x[:, :, 0] + w[:, 3] * x[:, :, 1], rtol=1e-14, atol=1e-15)


def test_conv_equals_library_convolution(oracle_mod):
    """Cropped full convolution with the reversed taps (numpy.convolve), then SiLU."""
    rng = np.random.default_rng(31)
    nb, nd, L = 2, 5, 37
    for K in (1, 2, 3, 4, 6):
        x = rng.standard_normal((nb, nd, L))
        w = rng.standard_normal((nd, K))
        b = rng.standard_normal(nd)
        out = oracle_mod.causal_conv1d(x, w, b, silu_flag=True)
        for bi in range(nb):
            for d in range(nd):
                pre = np.convolve(x[bi, d], w[d, ::-1])[:L] + b[d]
                np.testing.assert_allclose(out[bi, d], _silu(pre), rtol=1e-13, atol=1e-14)


def test_conv_impulse_response_is_the_taps(oracle_mod):
    """A unit impulse at t0 comes out as the taps, newest first: out[t0 + j] = w[K-1-j]."""
    nd, L, K, t0 = 4, 16, 4, 5
    rng = np.random.default_rng(32)
    w = rng.standard_normal((nd, K))
    x = np.zeros((1, nd, L))
    x[0, :, t0] = 1.0
    out = oracle_mod.causal_conv1d(x, w, None, silu_flag=False)[0]
    for j in range(L):
        want = w[:, K - 1 - (j - t0)] if 0 <= j - t0 < K else np.zeros(nd)
        np.testing.assert_array_equal(out[:, j], want)


def test_conv_is_causal_and_depthwise(oracle_mod):
    rng = np.random.default_rng(33)
    x = rng.standard_normal((1, 3, 20))
    w = rng.standard_normal((3, 4))
    b = rng.standard_normal(3)
    base = oracle_mod.causal_conv1d(x, w, b)
    fut = x.copy()
    fut[0, 1, 12] += 3.0            # a future token of channel 1
    moved = oracle_mod.causal_conv1d(fut, w, b)
    np.testing.assert_array_equal(moved[0, :, :12], base[0, :, :12])   # nothing earlier changes
    np.testing.assert_array_equal(moved[0, 0], base[0, 0])             # other channels never mix in
    np.testing.assert_array_equal(moved[0, 2], base[0, 2])
    assert np.all(moved[0, 1, 12:16] != base[0, 1, 12:16])             # the 4 outputs whose window holds it
    np.testing.assert_array_equal(moved[0, 1, 16:], base[0, 1, 16:])


def test_conv_width_one_is_pointwise(oracle_mod):
    rng = np.random.default_rng(34)
    x = rng.standard_normal((2, 3, 11))
    w = rng.standard_normal((3, 1))
    b = rng.standard_normal(3)
    out = oracle_mod.causal_conv1d(x, w, b, silu_flag=True)
    np.testing.assert_allclose(out, _silu(w[None, :, 0:1] * x + b[None, :, None]), rtol=1e-14, atol=1e-15)


def test_conv_window_steps_reproduce_sequence(oracle_mod):
    """From a zero window, the decode step (shift, insert, dot with the taps) gives the sequence
    convolution token by token, and the window ends holding the last K inputs."""
    rng = np.random.default_rng(35)
    nb, nd, L, K = 2, 3, 13, 4
    x = rng.standard_normal((nb, nd, L))
    w = rng.standard_normal((nd, K))
    b = rng.standard_normal(nd)
    seq = oracle_mod.causal_conv1d(x, w, b, silu_flag=True)
    win = np.zeros((nb, nd, K))
    for t in range(L):
        o, win = oracle_mod.conv_window_update(win, x[:, :, t], w, b, silu_flag=True)
        np.testing.assert_allclose(o, seq[:, :, t], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(win, x[:, :, L - K:])


# ------------------------------------------------------------------ backward scan
# The backward is pinned to the forward oracle itself, which the pins above tie to the pages: every
# gradient equals the central finite difference of J = sum(dout * out) in fp64.
def _fd_inputs(seed, nb=2, nd=3, L=6, N=4):
    rng = np.random.default_rng(seed)
    return {"u": rng.standard_normal((nb, nd, L)), "delta": 0.5 * rng.standard_normal((nb, nd, L)),
            "A": -np.exp(rng.standard_normal((nd, N))), "B": rng.standard_normal((nb, L, N)),
            "C": rng.standard_normal((nb, L, N)), "D": rng.standard_normal(nd), "z": rng.standard_normal((nb, nd, L)),
            "delta_bias": 0.3 * rng.standard_normal(nd)}, rng.standard_normal((nb, nd, L))


def _fd_check(oracle_mod, inp, dout, softplus, eps=1e-6):
    grads = oracle_mod.scan_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                inp["delta_bias"], dout=dout, softplus_flag=softplus)

    def J(x):
        out, _ = oracle_mod.scan_fwd(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                                     softplus_flag=softplus)
        return float(np.sum(out * dout))

    names = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
             "delta_bias": "ddelta_bias"}
    for key, gname in names.items():
        if inp[key] is None:
            assert grads[gname] is None
            continue
        fd = np.zeros_like(inp[key])
        for idx in np.ndindex(inp[key].shape):
            hi = {k: (v.copy() if v is not None else None) for k, v in inp.items()}
            lo = {k: (v.copy() if v is not None else None) for k, v in inp.items()}
            hi[key][idx] += eps
            lo[key][idx] -= eps
            fd[idx] = (J(hi) - J(lo)) / (2 * eps)
        np.testing.assert_allclose(grads[gname], fd, rtol=1e-6, atol=1e-7, err_msg="gradient " + gname)


@pytest.mark.parametrize("softplus", [True, False])
def test_backward_matches_finite_differences(oracle_mod, softplus):
    inp, dout = _fd_inputs(40)
    if not softplus:  # keep every step positive without softplus (else the states grow and J is huge)
        inp["delta"] = np.abs(inp["delta"]) + 0.05
        inp["delta_bias"] = np.abs(inp["delta_bias"])
    _fd_check(oracle_mod, inp, dout, softplus)


def test_backward_without_optional_inputs(oracle_mod):
    inp, dout = _fd_inputs(41)
    inp["D"] = inp["z"] = inp["delta_bias"] = None
    _fd_check(oracle_mod, inp, dout, True)


def test_backward_is_linear_in_dout(oracle_mod):
    inp, d1 = _fd_inputs(42)
    d2 = np.random.default_rng(43).standard_normal(d1.shape)
    args = (inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"])
    g1 = oracle_mod.scan_bwd(*args, dout=d1)
    g2 = oracle_mod.scan_bwd(*args, dout=d2)
    g12 = oracle_mod.scan_bwd(*args, dout=2.0 * d1 - d2)
    for k in g1:
        np.testing.assert_allclose(g12[k], 2.0 * g1[k] - g2[k], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ Mamba-2 (SSD) scan
# "Beyond attention with Mamba, state space models and hybrids", section 8: with a scalar decay a
# per head, the scan's output is a masked attention, y_t = sum_{s<=t} (c_t . b_s) e^{a_{s+1}+...+a_t}
# x_s, and the practical algorithm splits the sequence into chunks (attention inside a chunk, the
# recurrence between chunks, in four steps). The pins below compute those two forms independently
# of the oracle's step-by-step loop.
def ssd_inputs(nb=1, L=150, H=3, P=8, N=16, G=None, seed=0, a_scale=0.3):
    """The shapes and distributions of section 8's check: x, b, c ~ N(0, 1), a = -U(0, 1) * 0.3."""
    rng = np.random.default_rng(seed)
    G = H if G is None else G
    x = rng.standard_normal((nb, L, H, P))
    a = -rng.random((nb, L, H)) * a_scale
    b = rng.standard_normal((nb, L, G, N))
    c = rng.standard_normal((nb, L, G, N))
    return x, a, b, c


def ssd_attention_form(x, a, b, c):
    """The masked attention of section 8, written out as a double sum over t and s."""
    nb, L, H, P = x.shape
    G = b.shape[2]
    y = np.zeros_like(x)
    for bi in range(nb):
        for h in range(H):
            g = h // (H // G)
            cum = np.concatenate([[0.0], np.cumsum(a[bi, :, h])])  # cum[t + 1] = a_0 + ... + a_t
            for t in range(L):
                for s in range(t + 1):
                    w = float(c[bi, t, g] @ b[bi, s, g]) * math.exp(cum[t + 1] - cum[s + 1])
                    y[bi, t, h] += w * x[bi, s, h]
    return y


def ssd_chunked_form(x, a, b, c, chunk, dtype=np.float64):
    """Section 8's four steps, per chunk of `chunk` tokens: (1) inside the chunk, attention masked by
    the decay; (2) the state the chunk leaves behind; (3) the recurrence between chunks; (4) what
    each position reads from the state entering its chunk. Returns (y, final state)."""
    x, a, b, c = (np.asarray(v, dtype=dtype) for v in (x, a, b, c))
    nb, L, H, P = x.shape
    G, N = b.shape[2], b.shape[3]
    y = np.zeros((nb, L, H, P), dtype=dtype)
    final = np.zeros((nb, H, P, N), dtype=dtype)
    for bi in range(nb):
        for h in range(H):
            g = h // (H // G)
            entering = np.zeros((P, N), dtype=dtype)  # step 3's state entering the chunk
            for t0 in range(0, L, chunk):
                t1 = min(L, t0 + chunk)
                ac = np.cumsum(a[bi, t0:t1, h])                              # a_{t0} + ... + a_t
                cb = c[bi, t0:t1, g] @ b[bi, t0:t1, g].T                     # c_t . b_s
                mask = np.tril(np.exp(ac[:, None] - ac[None, :]))            # e^{a_{s+1}+...+a_t}, s <= t
                xs = x[bi, t0:t1, h]
                inside = (cb * mask) @ xs                                    # step 1
                reads = np.exp(ac)[:, None] * (c[bi, t0:t1, g] @ entering.T)  # step 4
                y[bi, t0:t1, h] = inside + reads
                to_end = np.exp(ac[-1] - ac)                                 # e^{a_{s+1}+...+a_end}
                left = (xs * to_end[:, None]).T @ b[bi, t0:t1, g]            # step 2: sum_s w_s x_s b_s^T
                entering = np.exp(ac[-1]) * entering + left                  # step 3
            final[bi, h] = entering
    return y, final


def test_ssd_chunked_form_equals_the_loop(oracle_mod):
    """Section 8 checks its chunked algorithm against the step-by-step loop on x [1, 150, 3, 8],
    N = 16, chunks of 32. In fp64 the two agree to rounding, for every chunk size."""
    x, a, b, c = ssd_inputs()
    y, fin = oracle_mod.ssd_scan(x, a, b, c)
    for chunk in (1, 7, 32, 64, 150, 256):
        yc, fc = ssd_chunked_form(x, a, b, c, chunk)
        np.testing.assert_allclose(y, yc, rtol=1e-11, atol=1e-11, err_msg="chunk %d" % chunk)
        np.testing.assert_allclose(fin, fc, rtol=1e-11, atol=1e-11, err_msg="chunk %d final state" % chunk)


def test_ssd_within_the_pages_fp32_gap(oracle_mod):
    """The page prints 6.7e-06 for the largest gap between its chunked form (fp32, chunks of 32) and the
    loop on inputs of this shape and distribution. The chunked form evaluated in fp32 here stays within
    a few times that of the fp64 oracle."""
    x, a, b, c = ssd_inputs(seed=5)
    y, _ = oracle_mod.ssd_scan(x, a, b, c)
    y32, _ = ssd_chunked_form(x, a, b, c, 32, dtype=np.float32)
    gap = float(np.max(np.abs(y32.astype(np.float64) - y)))
    assert 0 < gap < 5e-5


def test_ssd_attention_form(oracle_mod):
    """The masked-attention form of section 8, term by term, on small ragged shapes with shared groups."""
    for (nb, L, H, P, N, G, seed) in ((1, 23, 2, 3, 5, 2, 1), (2, 17, 4, 2, 3, 2, 2), (1, 9, 3, 1, 4, 1, 3)):
        x, a, b, c = ssd_inputs(nb, L, H, P, N, G, seed)
        y, _ = oracle_mod.ssd_scan(x, a, b, c, nthreads=1)  # one thread runs every row in turn
        np.testing.assert_allclose(y, ssd_attention_form(x, a, b, c), rtol=1e-11, atol=1e-11)


def test_ssd_special_cases(oracle_mod):
    """No decay (a = 0): the state is a running sum, y_t = sum_{s<=t} (c_t . b_s) x_s. Full forgetting
    (a very negative): y_t = (c_t . b_t) x_t. One state number, one channel, constant inputs: the
    geometric series h_t = x b (1 - e^{a (t+1)}) / (1 - e^a)."""
    x, a, b, c = ssd_inputs(1, 20, 2, 3, 4, 1, 7)
    y0, _ = oracle_mod.ssd_scan(x, np.zeros_like(a), b, c)
    for t in range(20):
        want = sum(float(c[0, t, 0] @ b[0, s, 0]) * x[0, s] for s in range(t + 1))
        np.testing.assert_allclose(y0[0, t], want, rtol=1e-12, atol=1e-12)
    yf, fin = oracle_mod.ssd_scan(x, np.full_like(a, -800.0), b, c)
    for t in range(20):
        np.testing.assert_allclose(yf[0, t], float(c[0, t, 0] @ b[0, t, 0]) * x[0, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin[0], np.einsum("hp,n->hpn", x[0, -1], b[0, -1, 0]), rtol=1e-12)
    L, av, xv, bv, cv = 12, -0.4, 1.5, 0.7, 2.0
    y1, f1 = oracle_mod.ssd_scan(np.full((1, L, 1, 1), xv), np.full((1, L, 1), av), np.full((1, L, 1, 1), bv),
                                 np.full((1, L, 1, 1), cv))
    h = xv * bv * (1.0 - np.exp(av * (np.arange(L) + 1))) / (1.0 - np.exp(av))
    np.testing.assert_allclose(y1.reshape(L), cv * h, rtol=1e-13)
    assert f1.item() == pytest.approx(h[-1], rel=1e-13)


def test_ssd_groups_share_b_and_c(oracle_mod):
    """Heads of one group read the same b and c: the result equals per-head b, c repeated by group."""
    x, a, b, c = ssd_inputs(2, 30, 6, 4, 8, 2, 11)
    y, fin = oracle_mod.ssd_scan(x, a, b, c)
    rep = lambda v: np.repeat(v, 3, axis=2)
    y2, fin2 = oracle_mod.ssd_scan(x, a, rep(b), rep(c))
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(fin, fin2)


def test_ssd_matches_the_s6_scan_when_a_is_shared(oracle_mod):
    """A Mamba-2 head with one channel (P = 1) is the S6 scan of a channel whose A has the same value for
    every state number: x = Delta u, a = Delta A, b = B, c = C (softplus off, no skip, no gate)."""
    rng = np.random.default_rng(13)
    nb, nd, L, N = 2, 5, 40, 16
    u = rng.standard_normal((nb, nd, L))
    dt = rng.uniform(0.01, 0.5, size=(nb, nd, L))
    Ad = -rng.uniform(0.1, 2.0, size=nd)
    B = rng.standard_normal((nb, L, N))
    C = rng.standard_normal((nb, L, N))
    out, last = oracle_mod.scan_fwd(u, dt, np.repeat(Ad[:, None], N, axis=1), B, C, softplus_flag=False)
    x = (dt * u).transpose(0, 2, 1)[..., None]               # [nb, L, nd, 1]
    a = (dt * Ad[None, :, None]).transpose(0, 2, 1)          # [nb, L, nd]
    y, fin = oracle_mod.ssd_scan(x, a, B[:, :, None, :], C[:, :, None, :])
    np.testing.assert_allclose(y[..., 0].transpose(0, 2, 1), out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin[:, :, 0, :], last, rtol=1e-12, atol=1e-12)
