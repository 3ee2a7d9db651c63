#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

One step = one ssm_scan_fwd call (softplus step, discretisation, recurrence, readout, skip and
gate, final state) over one batch of seeded synthetic input, through the C ABI. Default workload:
the long-context scan, bf16 inputs with fp32 state (batch 1, d_inner 2048, N 16, L 65536), the
largest single-GPU configuration.

Inputs are resident in HBM before the timed region. Each step reads a different copy of the
inputs (a rotation whose total exceeds the 256 MB last-level cache), so a step streams its bytes
from HBM rather than from cache. Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload long|mamba2p8b|mamba130m|decode|...] [--hot]
    python bench.py --peaks     # what this device sustains: copy bandwidth, VALU and exp issue rates
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "selective-scan Gelem-steps/s (B·L·D·N) + % MI355X HBM peak, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
# MI355X published fp32 vector peak: 256 CUs x 128 FMA lanes per clock x 2 flops x 2.4 GHz (the
# plain v_fma_f32 issue rate with VGPR operands measured on this device is 2 clocks per wave64
# instruction per SIMD, i.e. this figure; see bench.py --peaks).
FP32_VECTOR_PEAK_TFLOPS = 157.3
# MI355X published dense matrix-core peaks, by the inputs' type (bf16 inputs; fp32 inputs)
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
# Minimal ALU work, in VALU issue slots (an FMA-class instruction = 1 slot; a transcendental issues at
# a quarter of that rate = 4 slots; one slot = 2 flop-equivalents at the peak above):
#   per element-step (b, d, t, n): the decay's argument Delta*A (1), its exponential (4), the write
#     B*(Delta u) (1), the recurrence FMA (1) and the readout FMA (1): 8 slots;
#   per (b, d, t), shared by the N states: bias add (1), softplus = exp (4) + log (4) + 3 ops,
#     Delta*u (1), skip FMA D*u (1), gate SiLU(z) = exp (4) + reciprocal (4) + 3 ops, the product
#     y*SiLU(z) (1): 27 slots.
SLOTS_PER_ELEMENT_STEP = 8.0
SLOTS_PER_TOKEN = 27.0
# The backward's minimal VALU work, same units:
#   per element-step: the decay recomputed once (mul + exp: 5), the state recomputed (write mul, decayed
#     state mul, add: 3), the adjoint lambda = a lambda' + C dy (mul + FMA: 2), and the gradient terms
#     q = lambda * (a h_prev) (1), dA += q Delta (1), the step's sum over states q A (1) and lambda B (1),
#     dB += lambda Delta u (1), dC += h dy (1): 16 slots;
#   per (b, d, t): softplus and its derivative (exp, log, reciprocal and 4 ops: 16), SiLU(z) and its
#     derivative (exp, reciprocal and 5 ops: 13), dy, du, ddelta, dz and dD terms (7): 36 slots.
SLOTS_PER_ELEMENT_STEP_BWD = 16.0
SLOTS_PER_TOKEN_BWD = 36.0
COPY_CALIBRATION_BYTES = 256 << 20  # source size of the plain copy that calibrates the HBM counters
_CSRC = "mamba_selective_scan_s6_amd/csrc/"
_SCAN_SOURCES = [_CSRC + f for f in ("scan_fwd.hip", "scan_common.hpp", "lookback.hpp", "ssm_device.hpp")]
# The sources each workload's kernels are built from: a measurement stays valid while they are unchanged.
KERNEL_SOURCES = {
    "scan": _SCAN_SOURCES,
    "decode": [_CSRC + "state_update.hip", _CSRC + "ssm_device.hpp"],
    "conv": [_CSRC + "conv1d.hip", _CSRC + "ssm_device.hpp"],
    "bwd": _SCAN_SOURCES + [_CSRC + "scan_bwd.hip"],
    "ssd": [_CSRC + "ssd.hip", _CSRC + "ssm_device.hpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
WORKLOADS = ("mamba130m", "mamba2p8b", "long")


def source_family(workload: str) -> str:
    if workload in WORKLOADS:
        return "scan"
    if workload == "decode":
        return "decode"
    if workload.startswith("conv"):
        return "conv"
    if workload.startswith("bwd"):
        return "bwd"
    return "ssd"


def kernel_hash(workload: str = "long") -> str:
    """Hash of the sources of the kernels a workload runs."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[source_family(workload)]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on the
    current sources of the workload's kernels (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload_key)
    if not ent or ent.get("kernel_sha") != kernel_hash(workload_key.replace("_hot", "")):
        return None
    return ent.get("bytes_per_launch")


def to_dev(a, device):
    import torch

    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def cpu_baseline(inp, cfg, max_seconds=15.0, max_passes=50):
    """Time the fp64 oracle (as it stands) on the same workload on this host's cores: whole passes
    over the workload, repeated for about max_seconds, median pass time."""
    import oracle

    oracle.build(force=False)
    f = W.inputs_f64(inp)
    threads = oracle.default_threads()
    times = []
    t_all = time.time()
    while len(times) < max_passes and (not times or (time.time() - t_all) < max_seconds):
        t0 = time.perf_counter()
        oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"], f["delta_bias"], nthreads=threads)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    return {"value": cfg.element_steps / t / 1e9, "unit": "Gelem-steps/s", "cores": threads, "kind": "oracle",
            "sample": "the whole workload (%dx%dx%dx%d, same seeded inputs), %d pass(es) in %.1f s, median %.3f s"
                      % (cfg.nb, cfg.nd, cfg.L, cfg.N, len(times), time.time() - t_all, t)}


def _calibration_lib():
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "mamba_selective_scan_s6_amd", "libssmcal.so"))
    lib.ssmcal_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.ssmcal_rate.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


def copy_calibration(device, reps=5):
    """A plain copy of known size (COPY_CALIBRATION_BYTES read, as many written) by the calibration
    library's copy_kernel, for scaling the FETCH_SIZE / WRITE_SIZE counters; run only under the
    counter profiler, after the timed region."""
    import torch

    lib = _calibration_lib()
    src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    grid = torch.cuda.get_device_properties(device).multi_processor_count * 32
    for _ in range(reps):
        lib.ssmcal_copy(src.data_ptr(), dst.data_ptr(), COPY_CALIBRATION_BYTES, grid,
                        torch.cuda.current_stream(device).cuda_stream)
    torch.cuda.synchronize()


# Kernel (substring of the profiler's kernel name) whose dispatches each workload's traffic entry covers.
# For the SSD, "ssd_" matches the three kernels of one step (segment states, carries, outputs).
# the kernels whose counters make up one step of each workload (a name, or a tuple of names)
_BWD_KERNELS = ("scan_fwd_kernel", "segment_carry_kernel", "grad_kernel", "reduce_bc_kernel", "reduce_channel_kernel")
TRAFFIC_KERNEL = {"ssd2p7b": "ssd_", "ssd130m": "ssd_", "long": "scan_fwd_kernel", "mamba2p8b": "scan_fwd_kernel",
                  "mamba130m": "scan_fwd_kernel",
                  "decode": "state_update_kernel", "conv130m": "causal_conv1d_kernel",
                  "conv2p8b": "causal_conv1d_kernel", "bwd130m": _BWD_KERNELS, "bwd2p8b": _BWD_KERNELS}


def _is_step_kernel(workload: str, name: str) -> bool:
    want = TRAFFIC_KERNEL[workload]
    return any(k in name for k in (want if isinstance(want, tuple) else (want,)))


def algorithmic_bytes(workload: str) -> int:
    """Bytes one launch of the workload's kernel must move at least (each input read once, each
    output written once)."""
    if workload == "decode":
        return W.DECODE_CONFIG.algorithmic_bytes_per_step()
    if workload in SSD_WORKLOADS:
        return W.SSD_CONFIGS[workload].algorithmic_bytes()
    if workload in CONV_WORKLOADS:
        cfg = W.SCAN_CONFIGS[CONV_WORKLOADS[workload]]
        return 2 * cfg.nb * cfg.nd * cfg.L * W.io_itemsize(cfg.io) + cfg.nd * (CONV_WIDTH + 1) * 4
    if workload in BWD_WORKLOADS:
        # the forward's inputs and dout read once; du, ddelta, dz (io dtype) and dB, dC (fp32) written
        # once, plus the small per-channel gradients
        cfg = W.SCAN_CONFIGS[BWD_WORKLOADS[workload]]
        es = W.io_itemsize(cfg.io)
        tok = cfg.nb * cfg.nd * cfg.L
        return (4 * tok * es + 2 * cfg.nb * cfg.L * cfg.N * es + 3 * tok * es + 2 * cfg.nb * cfg.L * cfg.N * 4
                + cfg.nd * (cfg.N + 4) * 4 * 2)
    return W.SCAN_CONFIGS[workload].algorithmic_bytes()


def record_traffic(workload: str, fetch_csv: str, write_csv: str, command: str) -> dict:
    """Write the HBM traffic of one workload into the traffic file, from two rocprofv3 counter runs of
    `bench.py --workload W --copy-calibration` (one with FETCH_SIZE, one with WRITE_SIZE; both in KiB
    per dispatch). Each counter is scaled by what it reads for the calibration copy, whose true bytes
    are known. No GPU is needed."""
    import csv

    def per_dispatch(path, counter):
        vals = {}
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                key = (row["Dispatch_Id"], row["Kernel_Name"])
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
        kern = {}  # kernel name -> its dispatches' values
        for (d, name), v in vals.items():
            if _is_step_kernel(workload, name):
                kern.setdefault(name, []).append(v)
        copy = [v for (d, name), v in vals.items() if "copy_kernel" in name and "rocclr" not in name]
        if not kern or not copy:
            raise SystemExit("%s: no %s or copy_kernel dispatches with %s" % (path, TRAFFIC_KERNEL[workload], counter))
        # a step that launches several kernels (the split SSD form) counts each one's median once
        return (sum(statistics.median(v) for v in kern.values()), statistics.median(copy),
                min(len(v) for v in kern.values()))

    fetch_kib, fetch_copy_kib, nf = per_dispatch(fetch_csv, "FETCH_SIZE")
    write_kib, write_copy_kib, nw = per_dispatch(write_csv, "WRITE_SIZE")
    fetch_scale = COPY_CALIBRATION_BYTES / 1024.0 / fetch_copy_kib
    write_scale = COPY_CALIBRATION_BYTES / 1024.0 / write_copy_kib
    fetch_b = fetch_kib * 1024.0 * fetch_scale
    write_b = write_kib * 1024.0 * write_scale
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[workload] = {
        "kernel": TRAFFIC_KERNEL[workload], "kernel_sha": kernel_hash(workload),
        "bytes_per_launch": fetch_b + write_b, "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
        "fetch_size_kib_per_dispatch": fetch_kib, "write_size_kib_per_dispatch": write_kib,
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "copy_calibration_bytes": COPY_CALIBRATION_BYTES, "dispatches": [nf, nw],
        "algorithmic_bytes_per_launch": algorithmic_bytes(workload),
        "traffic_over_algorithmic": (fetch_b + write_b) / algorithmic_bytes(workload),
        "command": command,
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec[workload]


def alu_slots(cfg):
    """Minimal VALU issue slots of one launch (see SLOTS_PER_ELEMENT_STEP, SLOTS_PER_TOKEN)."""
    return cfg.element_steps * SLOTS_PER_ELEMENT_STEP + cfg.nb * cfg.nd * cfg.L * SLOTS_PER_TOKEN


def roofline(nbytes, slots, kern_ms, traffic):
    """Roofline of the scan kernel for one launch: HBM (algorithmic bytes) and ALU (minimal VALU
    issue slots as fp32 flop-equivalents, 2 per slot); the bound reported is the one whose peak
    allows the smaller rate for this workload."""
    sec = kern_ms * 1e-3
    gbs = nbytes / sec / 1e9
    tflops = 2.0 * slots / sec / 1e12
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_alu = 2.0 * slots / (FP32_VECTOR_PEAK_TFLOPS * 1e12)
    hbm = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
    alu = {"bound": "alu", "achieved": tflops, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": tflops / FP32_VECTOR_PEAK_TFLOPS}
    main, other = (hbm, alu) if t_hbm >= t_alu else (alu, hbm)
    res = dict(main)
    res.update({"traffic": traffic, "kernel_avg_ms": kern_ms, "algorithmic_bytes_per_launch": nbytes,
                "alu_slots_per_launch": slots, "flop_eq_per_launch": 2.0 * slots, "other_bound": other})
    return res


def bench_scan(args, device):
    import torch

    import mamba_selective_scan_s6_amd as S

    cfg = W.SCAN_CONFIGS[args.workload]
    inp = W.make_config_inputs(cfg)
    base = {k: to_dev(inp[k], device) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    nbytes = cfg.algorithmic_bytes()
    copies = 1 if args.hot else max(2, int(np.ceil(3 * 256e6 / nbytes)))  # > 3x the 256 MB cache
    copies = min(copies, 16)
    sets = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()} for _ in range(copies - 1)]
    outs = [torch.empty_like(base["u"]) for _ in range(copies)]
    states = [torch.empty((cfg.nb, cfg.nd, cfg.N), dtype=torch.float32, device=device) for _ in range(copies)]

    def step(i):
        s = sets[i % copies]
        S.ssm_scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], s["delta_bias"],
                       softplus_flag=True, out=outs[i % copies], last_state=states[i % copies], zoh=args.zoh)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(device)
    # the timed span: K back-to-back steps (one kernel launch each) between two events recorded on
    # the stream the kernels run on; the kernel's average launch duration is the span / K
    span0, span1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    span0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    span1.record(stream)
    torch.cuda.synchronize()
    ms_step = span0.elapsed_time(span1) / args.steps
    kern_ms = ms_step
    traffic = measured_traffic(args.workload + ("_hot" if args.hot else ""))
    S.stream_check(device)  # raises if a launch's cross-workgroup wait timed out (its output invalid)
    if args.copy_calibration:
        copy_calibration(device)
    res = {
        "metric": METRIC,
        "value": cfg.element_steps / (ms_step * 1e-3) / 1e9,
        "unit": "Gelem-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.io, "data": "synthetic (seeded numpy PCG64; no dataset or weights)",
        "config": {"workload": cfg.name, "batch": cfg.nb, "dim": cfg.nd, "seqlen": cfg.L, "dstate": cfg.N,
                   "io_dtype": cfg.io, "input_copies_rotated": copies,
                   "discretisation": "exact zero-order hold" if args.zoh else "Euler input gain (Delta B)"},
        "roofline": roofline(nbytes, alu_slots(cfg), kern_ms, traffic),
        "hbm_peak_frac": (nbytes / (ms_step * 1e-3) / 1e9) / HBM_PEAK_GBS,
        "kernel_sha": kernel_hash(args.workload),
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(inp, cfg)
    return res


def bench_decode(args, device):
    import torch

    import mamba_selective_scan_s6_amd as S

    cfg = W.DECODE_CONFIG
    prm = W.make_decode_params(cfg)
    state = to_dev(prm["state0"], device)
    A, D = to_dev(prm["A"], device), to_dev(prm["D"], device)
    steps_in = [{k: to_dev(v, device) for k, v in W.make_decode_step(cfg.nb, cfg.nd, cfg.N, cfg.seed, s).items()}
                for s in range(min(cfg.steps, 32))]
    outs = [torch.empty_like(steps_in[0]["x"]) for _ in range(len(steps_in))]

    def step(i):
        t = steps_in[i % len(steps_in)]
        S.ssm_state_update(state, t["x"], t["delta"], A, t["B"], t["C"], D, t["z"], out=outs[i % len(steps_in)])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kern_ms = statistics.mean(a.elapsed_time(b) for a, b in ev)
    nbytes = algorithmic_bytes("decode")
    achieved = nbytes / (kern_ms * 1e-3) / 1e9

    # The persistent 33.5 MB state fits in the 256 MB last-level cache; for the HBM-resident rate the
    # same steps also run rotating over 8 states (268 MB), each step on the next state.
    cold_ms = None
    if not args.no_rotating:
        states = [state] + [state.clone() for _ in range(7)]
        cold = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            t = steps_in[i % len(steps_in)]
            cold[i][0].record(stream)
            S.ssm_state_update(states[i % 8], t["x"], t["delta"], A, t["B"], t["C"], D, t["z"], out=outs[i % len(steps_in)])
            cold[i][1].record(stream)
        torch.cuda.synchronize()
        cold_ms = statistics.mean(a.elapsed_time(b) for a, b in cold)
    if args.copy_calibration:
        copy_calibration(device)
    return {"metric": "decode state-update Gelem-steps/s (B·D·N per token), 1 GPU",
            "value": cfg.element_steps_per_step / (ms * 1e-3) / 1e9, "unit": "Gelem-steps/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded numpy PCG64)",
            "config": {"workload": cfg.name, "batch": cfg.nb, "dim": cfg.nd, "dstate": cfg.N},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("decode"),
                         "kernel_avg_ms": kern_ms, "algorithmic_bytes_per_launch": nbytes},
            "rotating_8_states": None if cold_ms is None else {
                "kernel_avg_ms": cold_ms, "achieved_GBs": nbytes / (cold_ms * 1e-3) / 1e9,
                "frac": nbytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "kernel_sha": kernel_hash(args.workload)}


CONV_WORKLOADS = {"conv130m": "mamba130m", "conv2p8b": "mamba2p8b"}  # scan shapes, width-4 conv + SiLU
CONV_WIDTH = 4


def bench_conv(args, device):
    """The causal depthwise convolution + SiLU that produces the scan's input, on a scan workload's
    shape (width 4, as in Mamba); bound by HBM."""
    import torch

    import mamba_selective_scan_s6_amd as S

    cfg = W.SCAN_CONFIGS[CONV_WORKLOADS[args.workload]]
    K = CONV_WIDTH
    rng = np.random.default_rng(cfg.seed + 100)
    x = to_dev(W.to_io(rng.standard_normal((cfg.nb, cfg.nd, cfg.L)), cfg.io), device)
    w = to_dev((0.5 * rng.standard_normal((cfg.nd, K))).astype(np.float32), device)
    b = to_dev((0.1 * rng.standard_normal(cfg.nd)).astype(np.float32), device)
    nbytes = algorithmic_bytes(args.workload)
    copies = max(2, int(np.ceil(3 * 256e6 / nbytes)))
    copies = min(copies, 16)
    xs = [x] + [x.clone() for _ in range(copies - 1)]
    outs = [torch.empty_like(x) for _ in range(copies)]

    def step(i):
        S.causal_conv1d(xs[i % copies], w, b, silu=True, out=outs[i % copies])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kern_ms = statistics.mean(a.elapsed_time(b_) for a, b_ in ev)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    if args.copy_calibration:
        copy_calibration(device)
    return {"metric": "causal conv1d + SiLU GB/s (algorithmic bytes), 1 GPU",
            "value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": cfg.io, "data": "synthetic (seeded numpy PCG64)",
            "config": {"workload": "causal conv1d width 4 on " + cfg.name, "batch": cfg.nb, "dim": cfg.nd,
                       "seqlen": cfg.L, "width": K, "input_copies_rotated": copies},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload),
                         "kernel_avg_ms": kern_ms, "algorithmic_bytes_per_launch": nbytes},
            "kernel_sha": kernel_hash(args.workload)}


BWD_WORKLOADS = {"bwd130m": "mamba130m", "bwd2p8b": "mamba2p8b"}  # backward scan on the scan shapes


def bench_bwd(args, device):
    """ssm_scan_bwd (forward recompute with checkpoints, adjoint, gradients) on a scan workload."""
    import torch

    import mamba_selective_scan_s6_amd as S

    cfg = W.SCAN_CONFIGS[BWD_WORKLOADS[args.workload]]
    inp = W.make_config_inputs(cfg)
    t = {k: to_dev(inp[k], device) for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    dout = to_dev(W.to_io(np.random.default_rng(cfg.seed + 200).standard_normal(inp["u"].shape), cfg.io), device)

    def step():
        S.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], dout=dout)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    S.stream_check(device)
    ms = e0.elapsed_time(e1) / args.steps
    if args.copy_calibration:
        copy_calibration(device)
    nbytes = algorithmic_bytes(args.workload)
    tok = cfg.nb * cfg.nd * cfg.L
    slots = cfg.element_steps * SLOTS_PER_ELEMENT_STEP_BWD + tok * SLOTS_PER_TOKEN_BWD
    return {"metric": "backward selective-scan Gelem-steps/s (B·L·D·N), 1 GPU",
            "value": cfg.element_steps / (ms * 1e-3) / 1e9, "unit": "Gelem-steps/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": cfg.io, "data": "synthetic (seeded numpy PCG64)",
            "config": {"workload": "backward of " + cfg.name, "batch": cfg.nb, "dim": cfg.nd, "seqlen": cfg.L,
                       "dstate": cfg.N},
            "roofline": dict(roofline(nbytes, slots, ms, measured_traffic(args.workload)),
                             scope="the whole backward pass (its 5 kernels), per call"),
            "kernel_sha": kernel_hash(args.workload)}


SSD_WORKLOADS = ("ssd130m", "ssd2p7b")


def ssd_mfma_flops(cfg) -> float:
    """Matrix-core flops of one call in the chunked form with chunks of T = 32 tokens: per (batch row,
    head, chunk) the causal score tiles (T/16 (T/16 + 1) / 2 tiles of 16 x 16 x N), the masked scores
    times x (the same tiles, 16 x 16 x P each), the state's readout (T x N x P) and the chunk's state
    update (N x T x P), 2 flops per multiply-add. The split form's second pass over the state updates of
    all segments but the last is not counted (it is the implementation's, not the algorithm's)."""
    T = 32
    tiles = (T // 16) * (T // 16 + 1) // 2
    per_chunk = 2.0 * (tiles * 256 * cfg.N + tiles * 256 * cfg.P + 2 * T * cfg.N * cfg.P)
    return per_chunk * cfg.nb * cfg.H * ((cfg.L + T - 1) // T)


def bench_ssd(args, device):
    """Mamba-2's scan (ssm_ssd_scan) on a layer's shape; bound by HBM at the published peaks."""
    import torch

    import mamba_selective_scan_s6_amd as S

    cfg = W.SSD_CONFIGS[args.workload]
    inp = W.make_ssd_config_inputs(cfg)
    base = {k: to_dev(inp[k], device) for k in ("x", "a", "b", "c")}
    nbytes = cfg.algorithmic_bytes()
    copies = max(2, int(np.ceil(3 * 256e6 / nbytes)))  # rotate past the 256 MB last-level cache
    copies = min(copies, 16)
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
    ys = [torch.empty(tuple(base["x"].shape), dtype=base["x"].dtype, device=device) for _ in range(copies)]
    fs = [torch.empty((cfg.nb, cfg.H, cfg.P, cfg.N), dtype=torch.float32, device=device) for _ in range(copies)]

    def step(i):
        s = sets[i % copies]
        S.ssd_scan(s["x"], s["a"], s["b"], s["c"], y=ys[i % copies], final_state=fs[i % copies])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    sec = ms * 1e-3
    gbs = nbytes / sec / 1e9
    flops = ssd_mfma_flops(cfg)
    mfma_peak = MFMA_PEAK_TFLOPS[cfg.io]
    if args.copy_calibration:
        copy_calibration(device)
    return {"metric": "Mamba-2 SSD scan Gelem-steps/s (B·L·H·P·N state updates), 1 GPU",
            "value": cfg.element_steps / sec / 1e9, "unit": "Gelem-steps/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": cfg.io, "data": "synthetic (seeded numpy PCG64)",
            "config": {"workload": cfg.name, "batch": cfg.nb, "seqlen": cfg.L, "heads": cfg.H, "headdim": cfg.P,
                       "dstate": cfg.N, "ngroups": cfg.G, "input_copies_rotated": copies},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(args.workload),
                         "kernel_avg_ms": ms, "algorithmic_bytes_per_launch": nbytes,
                         "other_bound": {"bound": "mfma", "achieved": flops / sec / 1e12, "peak": mfma_peak,
                                         "unit": "TFLOP/s", "frac": flops / sec / 1e12 / mfma_peak,
                                         "flops_per_launch": flops}},
            "kernel_sha": kernel_hash(args.workload)}


def bench_peaks(args, device):
    """What this device sustains, measured with the calibration kernels (libssmcal.so): a plain copy
    (HBM), fp32 FMA chains (VALU issue rate), exponential chains (transcendental issue rate) and the
    scan's element-step mix. The published figures the rooflines use are reported beside them."""

    import torch

    lib = _calibration_lib()
    props = torch.cuda.get_device_properties(device)
    cus = props.multi_processor_count
    stream = torch.cuda.current_stream(device)
    sh = stream.cuda_stream

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = None
        for _ in range(reps):
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    copy = {}
    for per_cu in (8, 32, 128, 512):
        grid = cus * per_cu
        ms = timed(lambda: lib.ssmcal_copy(src.data_ptr(), dst.data_ptr(), nbytes, grid, sh))
        copy[grid] = 2.0 * nbytes / (ms * 1e-3) / 1e9
    del src, dst
    grid = cus * 8  # 8 workgroups of 4 waves per CU: 8 waves per SIMD
    out = torch.empty(grid * 256, dtype=torch.float32, device=device)
    iters = 4000
    lanes = grid * 256
    rates = {}
    for kind, name, per_iter in ((0, "fma", 32), (1, "exp", 8), (2, "element_step", 16)):
        ms = timed(lambda: lib.ssmcal_rate(kind, out.data_ptr(), iters, grid, sh))
        rates[name] = lanes * iters * per_iter / (ms * 1e-3)
    clk = 2.4e9
    simd_clk = cus * 4 * clk  # SIMD-clocks per second at the published clock
    res = {
        "metric": "device peaks (measured on this GPU; published figures beside)", "n_gpus": 1,
        "device": props.name, "compute_units": cus,
        "copy_GBps_best": max(copy.values()), "copy_GBps_by_grid": copy, "hbm_published_GBps": HBM_PEAK_GBS,
        "fma_lane_ops_per_s": rates["fma"], "fma_TFLOPs": 2 * rates["fma"] / 1e12,
        "fp32_vector_published_TFLOPs": FP32_VECTOR_PEAK_TFLOPS,
        "fma_clocks_per_wave64_instruction_per_SIMD_at_2.4GHz": simd_clk * 64 / rates["fma"],
        "exp_lane_ops_per_s": rates["exp"],
        "exp_clocks_per_wave64_instruction_per_SIMD_at_2.4GHz": simd_clk * 64 / rates["exp"],
        "element_steps_per_s": rates["element_step"],
        "element_step_clocks_per_wave64_per_SIMD_at_2.4GHz": simd_clk * 64 / rates["element_step"],
        "note": "element step = decay argument (mul), exp2, write (mul), recurrence FMA, readout FMA, exps grouped by 4",
    }
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="long",
                    choices=sorted(WORKLOADS) + ["decode"] + sorted(CONV_WORKLOADS) + sorted(BWD_WORKLOADS)
                    + list(SSD_WORKLOADS))
    ap.add_argument("--hot", action="store_true", help="reuse one input copy (cache-resident)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--zoh", action="store_true", help="scan with the exact zero-order-hold input gain")
    ap.add_argument("--no-rotating", action="store_true", help="decode: skip the leg that rotates over 8 states")
    ap.add_argument("--peaks", action="store_true", help="measure copy bandwidth and VALU / exp issue rates")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a %d MiB plain copy (for scaling HBM counters)" % (COPY_CALIBRATION_BYTES >> 20))
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store --workload's HBM traffic from two rocprofv3 counter CSVs (FETCH_SIZE, WRITE_SIZE) "
                         "in profiles/traffic.json; no GPU needed")
    ap.add_argument("--command", default="", help="with --record-traffic: the profiler command that made the CSVs")
    args = ap.parse_args()
    if args.record_traffic:
        print(json.dumps(record_traffic(args.workload, *args.record_traffic, args.command)), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    device = torch.device("cuda:0")
    if args.peaks:
        res = bench_peaks(args, device)
    elif args.workload == "decode":
        res = bench_decode(args, device)
    elif args.workload in CONV_WORKLOADS:
        res = bench_conv(args, device)
    elif args.workload in BWD_WORKLOADS:
        res = bench_bwd(args, device)
    elif args.workload in SSD_WORKLOADS:
        res = bench_ssd(args, device)
    else:
        res = bench_scan(args, device)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
