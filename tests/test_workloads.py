"""The seeded input module: exact io rounding, determinism, shapes."""
import numpy as np

import workloads as W


def _bf16_neighbours(x):
    """The two bf16 values bracketing x (by stepping the fp32 bit pattern's top half)."""
    f = np.float32(x)
    hi16 = np.uint32(f.view(np.uint32)) >> np.uint32(16)
    lo = W.bf16_bits_to_f64(np.array([hi16], dtype=np.uint16))[0]
    up = W.bf16_bits_to_f64(np.array([hi16 + 1], dtype=np.uint16))[0]
    down = W.bf16_bits_to_f64(np.array([hi16 - 1], dtype=np.uint16))[0]
    return lo, up, down


def test_bf16_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-3, rng.standard_normal(2000) * 1e4])
    bits = W.f64_to_bf16_bits(x)
    got = W.bf16_bits_to_f64(bits)
    for xi, gi in zip(x[:3000], got[:3000]):
        lo, up, down = _bf16_neighbours(xi)
        best = min((abs(c - xi), c) for c in (lo, up, down))[0]
        assert abs(gi - xi) == best
    # relative error bound 2^-8 (half an ulp) for RNE into 8 significant bits
    assert np.all(np.abs(got - x) <= np.abs(x) * 2.0 ** -8 + 1e-300)


def test_bf16_ties_go_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even pattern (1.0).
    assert W.bf16_bits_to_f64(W.f64_to_bf16_bits(np.array([1 + 2.0 ** -8])))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6 (even mantissa).
    assert W.bf16_bits_to_f64(W.f64_to_bf16_bits(np.array([1 + 3 * 2.0 ** -8])))[0] == 1 + 2.0 ** -6
    # fp64 values just above the tie round up (no double rounding through fp32).
    assert W.bf16_bits_to_f64(W.f64_to_bf16_bits(np.array([1 + 2.0 ** -8 + 2.0 ** -40])))[0] == 1 + 2.0 ** -7


def test_generators_are_deterministic_and_shaped():
    a = W.make_scan_inputs(2, 8, 33, 16, W.BF16, seed=5)
    b = W.make_scan_inputs(2, 8, 33, 16, W.BF16, seed=5)
    for k in ("u", "delta", "z", "B", "C", "A", "D", "delta_bias"):
        np.testing.assert_array_equal(a[k], b[k])
    assert a["u"].shape == (2, 8, 33) and a["u"].dtype == np.uint16
    assert a["B"].shape == (2, 33, 16)
    assert a["A"].shape == (8, 16) and a["A"].dtype == np.float32
    np.testing.assert_array_equal(a["A"][3], -(np.arange(16) + 1.0))
    c = W.make_scan_inputs(2, 8, 33, 16, W.BF16, seed=6)
    assert not np.array_equal(a["u"], c["u"])
    f = W.make_scan_inputs(1, 4, 10, 16, W.F32, seed=1)
    assert f["u"].dtype == np.float32


def test_dt_bias_recipe_range():
    inp = W.make_scan_inputs(1, 4096, 1, 16, W.F32, seed=0)
    assert 1e-3 <= inp["dt"].min() and inp["dt"].max() <= 1e-1
    # softplus(bias) = dt, written out from the definition log(1 + e^x)
    sp = np.log1p(np.exp(inp["delta_bias"].astype(np.float64)))
    np.testing.assert_allclose(sp, inp["dt"], rtol=1e-6)


def test_config_sizes():
    c1 = W.SCAN_CONFIGS["mamba130m"]
    assert c1.element_steps == 50331648
    assert c1.algorithmic_bytes() == 50802688
    assert W.SCAN_CONFIGS["mamba2p8b"].algorithmic_bytes() == 337747968
    assert W.SCAN_CONFIGS["long"].algorithmic_bytes() == 1078214656
    assert W.DECODE_CONFIG.algorithmic_bytes_per_step() == 71864320


def test_rows_subset_matches_slices():
    inp = W.make_scan_inputs(2, 10, 12, 16, W.F32, seed=2)
    sub = W.rows_subset(inp, [1, 7])
    np.testing.assert_array_equal(sub["u"], inp["u"][:, [1, 7]])
    np.testing.assert_array_equal(sub["A"], inp["A"][[1, 7]])
    np.testing.assert_array_equal(sub["delta_bias"], inp["delta_bias"][[1, 7]])
    assert sub["nd"] == 2
