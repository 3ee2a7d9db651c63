"""Seeded synthetic inputs for the selective scan and its decode step.

This module holds the workload recipes only: shapes, distributions, seeds and the exact
rounding of fp64 draws to the io dtype. It holds none of the method's arithmetic, and it is
the one piece of code that both the oracle side (tests) and the HIP side (tests, benchmark)
use, so that both see bit-identical inputs.

Recipes (no dataset is involved; the pages time their scan on random tensors of mamba-130m
width, "Beyond attention with Mamba, state space models and hybrids", section 6):
  * A[d, n] = -(n + 1) (the S4D-real initialisation; A = -exp(A_log) with A_log = log(n + 1)).
  * dt_d log-uniform in [1e-3, 1e-1]; delta_bias_d = softplus^-1(dt_d) = dt + log(-expm1(-dt)),
    so that softplus(bias) = dt (the dt initialisation of the same page, section 11).
  * delta_raw = scale * N(0, 1) with scale 0.5 (1.0 for the long-context workload).
  * u, z, B, C ~ N(0, 1); D = 1 or D ~ U(0.5, 1.5).
  * decode: state0 ~ N(0, 0.1^2) fp32; per step x, z, delta_raw, B, C ~ N(0, 1).
Every value is drawn in fp64 from numpy's PCG64 and rounded to nearest-even into fp32 or bf16.
bf16 tensors are carried as uint16 bit patterns.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

F32 = "f32"
BF16 = "bf16"


# ----------------------------------------------------------------------------- bf16 bits
def f64_to_bf16_bits(x) -> np.ndarray:
    """Round fp64 values to bfloat16 (nearest, ties to even) in one step; return uint16 bits.

    Exact for every finite value inside bf16's normal range (the only values drawn here)."""
    b = np.ascontiguousarray(x, dtype=np.float64).view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    b = b + np.uint64((1 << 44) - 1) + lsb
    b = b & ~np.uint64((1 << 45) - 1)
    f = b.view(np.float64).astype(np.float32)  # at most 8 significant bits: exact
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def to_io(x64, io: str) -> np.ndarray:
    """fp64 -> io representation (float32 array, or uint16 bf16 bits)."""
    if io == F32:
        return np.asarray(x64, dtype=np.float64).astype(np.float32)
    if io == BF16:
        return f64_to_bf16_bits(x64)
    raise ValueError("unknown io dtype %r" % io)


def io_to_f64(a, io: str) -> np.ndarray:
    if io == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if io == BF16:
        return bf16_bits_to_f64(a)
    raise ValueError("unknown io dtype %r" % io)


def io_itemsize(io: str) -> int:
    return 4 if io == F32 else 2


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()[:16]


# ----------------------------------------------------------------------------- configs
@dataclass(frozen=True)
class ScanConfig:
    name: str
    nb: int
    nd: int
    L: int
    N: int
    io: str
    delta_scale: float
    d_uniform: bool
    seed: int

    @property
    def element_steps(self) -> int:
        return self.nb * self.L * self.nd * self.N

    def algorithmic_bytes(self, with_state: bool = True) -> int:
        """Bytes a scan must move at least once: u, delta, z read and out written
        ([nb, nd, L] each, io dtype), B and C ([nb, L, N], io dtype), A ([nd, N] fp32),
        D and delta_bias ([nd] fp32 each), last_state written ([nb, nd, N] fp32)."""
        s = io_itemsize(self.io)
        per_row = 4 * self.nb * self.nd * self.L * s
        bc = 2 * self.nb * self.L * self.N * s
        params = self.nd * self.N * 4 + 2 * self.nd * 4
        state = self.nb * self.nd * self.N * 4 if with_state else 0
        return per_row + bc + params + state


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    nb: int
    nd: int
    N: int
    steps: int
    seed: int

    @property
    def element_steps_per_step(self) -> int:
        return self.nb * self.nd * self.N

    def algorithmic_bytes_per_step(self) -> int:
        """state read + written (fp32), x, delta, z read and out written (bf16, [nb, nd]),
        B and C (bf16, [nb, N]), A (fp32, [nd, N]), D (fp32, [nd])."""
        st = 2 * self.nb * self.nd * self.N * 4
        rows = 4 * self.nb * self.nd * 2
        bc = 2 * self.nb * self.N * 2
        return st + rows + bc + self.nd * self.N * 4 + self.nd * 4


SCAN_CONFIGS = {
    "toy": ScanConfig("toy S6 scan fp32 (1x64x128, N16)", 1, 64, 128, 16, F32, 0.5, False, 0),
    "mamba130m": ScanConfig("mamba-130m layer fp32 (1x1536x2048, N16)", 1, 1536, 2048, 16, F32, 0.5, True, 1),
    "mamba2p8b": ScanConfig("mamba-2.8b-like layer bf16 (4x5120x2048, N16)", 4, 5120, 2048, 16, BF16, 0.5, True, 2),
    "long": ScanConfig("long-context bf16 (1x2048x65536, N16)", 1, 2048, 65536, 16, BF16, 1.0, True, 3),
}
DECODE_CONFIG = DecodeConfig("decode bf16 (64x8192, N16, 256 steps)", 64, 8192, 16, 256, 4)


@dataclass(frozen=True)
class SsdConfig:
    """A Mamba-2 layer's scan: batch, sequence, heads, head dimension P, state N, groups sharing b, c."""
    name: str
    nb: int
    L: int
    H: int
    P: int
    N: int
    G: int
    io: str
    seed: int

    @property
    def element_steps(self) -> int:
        """State numbers updated per call: every token updates each head's P x N state."""
        return self.nb * self.L * self.H * self.P * self.N

    def algorithmic_bytes(self) -> int:
        """x read and y written ([nb, L, H, P], io dtype), b and c read ([nb, L, G, N], io dtype), a read
        ([nb, L, H] fp32), the final state written ([nb, H, P, N] fp32)."""
        s = io_itemsize(self.io)
        return (2 * self.nb * self.L * self.H * self.P * s + 2 * self.nb * self.L * self.G * self.N * s
                + self.nb * self.L * self.H * 4 + self.nb * self.H * self.P * self.N * 4)


SSD_CONFIGS = {
    "ssd130m": SsdConfig("mamba2-130m layer fp32 (1x2048, 24 heads x 64, N128)", 1, 2048, 24, 64, 128, 1, F32, 10),
    "ssd2p7b": SsdConfig("mamba2-2.7b-like layer bf16 (4x2048, 80 heads x 64, N128)", 4, 2048, 80, 64, 128, 1, BF16, 11),
}


# ----------------------------------------------------------------------------- generators
_BLOCK = 1 << 23  # draw big tensors in blocks of 8M values to bound host memory


def _normal_io(rng: np.random.Generator, shape, scale: float, io: str) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if io == F32 else np.uint16)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        x = rng.standard_normal(e - s)
        if scale != 1.0:
            x *= scale
        out[s:e] = to_io(x, io)
    return out.reshape(shape)


def s4d_real_A(nd: int, N: int) -> np.ndarray:
    """A[d, n] = -(n + 1), fp32."""
    return np.tile(-(np.arange(N, dtype=np.float64) + 1.0), (nd, 1)).astype(np.float32)


def softplus_inverse(y) -> np.ndarray:
    """The bias that softplus maps to y: y + log(-expm1(-y)) (used to set delta_bias from dt)."""
    y = np.asarray(y, dtype=np.float64)
    return y + np.log(-np.expm1(-y))


def make_scan_inputs(nb: int, nd: int, L: int, N: int, io: str, seed: int, delta_scale: float = 0.5,
                     d_uniform: bool = True, with_z: bool = True) -> dict:
    """Seeded scan inputs in io representation. Draw order is fixed:
    dt, D (if uniform), u, delta_raw, z, B, C."""
    rng = np.random.default_rng(seed)
    A = s4d_real_A(nd, N)
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=nd))
    delta_bias = softplus_inverse(dt).astype(np.float32)
    D = rng.uniform(0.5, 1.5, size=nd).astype(np.float32) if d_uniform else np.ones(nd, np.float32)
    u = _normal_io(rng, (nb, nd, L), 1.0, io)
    delta = _normal_io(rng, (nb, nd, L), delta_scale, io)
    z = _normal_io(rng, (nb, nd, L), 1.0, io)
    B = _normal_io(rng, (nb, L, N), 1.0, io)
    C = _normal_io(rng, (nb, L, N), 1.0, io)
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z if with_z else None, delta_bias=delta_bias,
                io=io, nb=nb, nd=nd, L=L, N=N, dt=dt)


def make_ssd_inputs(nb: int, L: int, H: int, P: int, N: int, G: int, io: str, seed: int, layer: bool = True) -> dict:
    """Seeded inputs of a Mamba-2 scan in io representation (a stays fp32). layer=True: a Mamba-2 layer's
    distributions, x = u * step and a = step * A with u ~ N(0, 1), A = -U(1, 16) per head and
    step = softplus(0.5 N(0, 1) + bias), the bias putting the typical step between 1e-3 and 1e-1 per
    head; layer=False: the check of section 8 of "Beyond attention with Mamba ...", x ~ N(0, 1) and
    a = -0.3 U(0, 1). b, c ~ N(0, 1) in both. Draw order is fixed: (A, bias), u or x, raw step or a, b, c."""
    rng = np.random.default_rng(seed)
    if layer:
        A = -rng.uniform(1.0, 16.0, size=H)
        bias = softplus_inverse(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=H)))
        u = rng.standard_normal((nb, L, H, P))
        r = 0.5 * rng.standard_normal((nb, L, H)) + bias
        step = np.maximum(r, 0.0) + np.log1p(np.exp(-np.abs(r)))
        x = to_io((u * step[..., None]).reshape(-1), io).reshape(nb, L, H, P)
        a = (step * A).astype(np.float32)
    else:
        x = _normal_io(rng, (nb, L, H, P), 1.0, io)
        a = (-0.3 * rng.random((nb, L, H))).astype(np.float32)
    b = _normal_io(rng, (nb, L, G, N), 1.0, io)
    c = _normal_io(rng, (nb, L, G, N), 1.0, io)
    return dict(x=x, a=a, b=b, c=c, io=io, nb=nb, L=L, H=H, P=P, N=N, G=G)


def make_ssd_config_inputs(cfg: "SsdConfig", seed: int | None = None) -> dict:
    return make_ssd_inputs(cfg.nb, cfg.L, cfg.H, cfg.P, cfg.N, cfg.G, cfg.io, cfg.seed if seed is None else seed)


def ssd_inputs_f64(inp: dict) -> dict:
    """float64 views of an SSD input set (exact), for the oracle."""
    io = inp["io"]
    return {k: io_to_f64(inp[k], io) if k != "a" else np.asarray(inp["a"], dtype=np.float64) for k in ("x", "a", "b", "c")}


def make_config_inputs(cfg: ScanConfig, seed: int | None = None) -> dict:
    return make_scan_inputs(cfg.nb, cfg.nd, cfg.L, cfg.N, cfg.io, cfg.seed if seed is None else seed,
                            cfg.delta_scale, cfg.d_uniform)


def make_decode_params(cfg: DecodeConfig, seed: int | None = None) -> dict:
    """A, D and the initial fp32 state (state0 ~ N(0, 0.1^2))."""
    rng = np.random.default_rng([cfg.seed if seed is None else seed, 0xDEC0DE])
    state0 = (0.1 * rng.standard_normal((cfg.nb, cfg.nd, cfg.N))).astype(np.float32)
    return dict(A=s4d_real_A(cfg.nd, cfg.N), D=np.ones(cfg.nd, np.float32), state0=state0)


def make_decode_step(nb: int, nd: int, N: int, seed: int, step: int) -> dict:
    """One decode token's inputs (bf16 bits): x, delta_raw, z [nb, nd]; B, C [nb, N].
    Each step has its own stream, so any step can be regenerated on its own."""
    rng = np.random.default_rng([seed, step])
    return dict(x=_normal_io(rng, (nb, nd), 1.0, BF16), delta=_normal_io(rng, (nb, nd), 1.0, BF16),
                z=_normal_io(rng, (nb, nd), 1.0, BF16), B=_normal_io(rng, (nb, N), 1.0, BF16),
                C=_normal_io(rng, (nb, N), 1.0, BF16))


def rows_subset(inp: dict, channels) -> dict:
    """The same inputs restricted to some channels (every batch row kept). Rows of the scan
    are independent, so the oracle on the subset gives exactly those rows of the full result."""
    ch = np.asarray(channels)
    sub = dict(inp)
    for k in ("u", "delta", "z"):
        if inp.get(k) is not None:
            sub[k] = np.ascontiguousarray(inp[k][:, ch, :])
    sub["A"] = np.ascontiguousarray(inp["A"][ch])
    for k in ("D", "delta_bias"):
        if inp.get(k) is not None:
            sub[k] = np.ascontiguousarray(inp[k][ch])
    sub["nd"] = len(ch)
    return sub


def inputs_f64(inp: dict) -> dict:
    """float64 views of every tensor (exact), for the oracle."""
    io = inp["io"]
    out = {}
    for k in ("u", "delta", "z", "B", "C"):
        out[k] = None if inp.get(k) is None else io_to_f64(inp[k], io)
    for k in ("A", "D", "delta_bias"):
        out[k] = None if inp.get(k) is None else np.asarray(inp[k], dtype=np.float64)
    return out
