#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

One step = one ssm_scan_fwd call (softplus step, discretisation, recurrence, readout, skip and
gate, final state) over one batch of seeded synthetic input, through the C ABI. Default workload:
the mamba-130m layer shape in fp32 (batch 1, d_inner 1536, N 16, L 2048).

Inputs are resident in HBM before the timed region. Each step reads a different copy of the
inputs (a rotation whose total exceeds the 256 MB last-level cache), so a step streams its bytes
from HBM rather than from cache. Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload mamba130m|mamba2p8b|long|decode] [--hot]
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
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X published fp32 vector peak (256 CUs at 2.4 GHz)
# Minimal VALU work of one element-step, in fp32 flop-equivalents: the step-times-A multiply, the
# B (step x) multiply, the recurrence FMA and the readout FMA (4 FMA issue slots), plus one exp,
# which issues at a quarter of the FMA rate (4 slots): 8 FMA slots = 16 flop-equivalents.
FLOP_EQ_PER_ELEMENT_STEP = 16.0
COPY_CALIBRATION_BYTES = 256 << 20  # source size of the plain copy that calibrates the HBM counters
KERNEL_SOURCES = ["mamba_selective_scan_s6_amd/csrc/scan_fwd.hip", "mamba_selective_scan_s6_amd/csrc/ssm_device.hpp",
                  "mamba_selective_scan_s6_amd/csrc/state_update.hip", "mamba_selective_scan_s6_amd/csrc/conv1d.hip",
                  "mamba_selective_scan_s6_amd/csrc/scan_common.hpp", "mamba_selective_scan_s6_amd/csrc/scan_bwd.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
WORKLOADS = ("mamba130m", "mamba2p8b", "long")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on the
    current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload_key)
    if not ent or ent.get("kernel_sha") != kernel_hash():
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


def cpu_baseline(inp, cfg, max_seconds=10.0, max_passes=50):
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


def copy_calibration(device, reps=5):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
    (run only under the counter profiler; not part of the timed region)."""
    import torch

    n = COPY_CALIBRATION_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device=device)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()


def roofline(nbytes, element_steps, kern_ms, traffic):
    """Roofline of the scan kernel for one launch: HBM (algorithmic bytes) and VALU (flop-
    equivalents); the bound reported is the one that allows the smaller rate for this workload."""
    sec = kern_ms * 1e-3
    gbs = nbytes / sec / 1e9
    tflops = element_steps * FLOP_EQ_PER_ELEMENT_STEP / sec / 1e12
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_alu = element_steps * FLOP_EQ_PER_ELEMENT_STEP / (FP32_VECTOR_PEAK_TFLOPS * 1e12)
    hbm = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
    alu = {"bound": "alu", "achieved": tflops, "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": tflops / FP32_VECTOR_PEAK_TFLOPS}
    main, other = (hbm, alu) if t_hbm >= t_alu else (alu, hbm)
    res = dict(main)
    res.update({"traffic": traffic, "kernel_avg_ms": kern_ms, "algorithmic_bytes_per_launch": nbytes,
                "flop_eq_per_launch": element_steps * FLOP_EQ_PER_ELEMENT_STEP, "other_bound": other})
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
    # the timed span: K back-to-back steps between two events
    span0, span1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    span0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    span1.record(stream)
    torch.cuda.synchronize()
    ms_step = span0.elapsed_time(span1) / args.steps
    # the kernel's own duration: the same steps again, each between two events on its stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(args.warmup + args.steps + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kern_ms = statistics.mean(a.elapsed_time(b) for a, b in ev)
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
        "roofline": roofline(nbytes, cfg.element_steps, kern_ms, traffic),
        "hbm_peak_frac": (nbytes / (ms_step * 1e-3) / 1e9) / HBM_PEAK_GBS,
        "kernel_sha": kernel_hash(),
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
    nbytes = cfg.algorithmic_bytes_per_step()
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
            "kernel_sha": kernel_hash()}


CONV_WORKLOADS = {"conv130m": "mamba130m", "conv2p8b": "mamba2p8b"}  # scan shapes, width-4 conv + SiLU


def bench_conv(args, device):
    """The causal depthwise convolution + SiLU that produces the scan's input, on a scan workload's
    shape (width 4, as in Mamba); bound by HBM."""
    import torch

    import mamba_selective_scan_s6_amd as S

    cfg = W.SCAN_CONFIGS[CONV_WORKLOADS[args.workload]]
    K = 4
    rng = np.random.default_rng(cfg.seed + 100)
    x = to_dev(W.to_io(rng.standard_normal((cfg.nb, cfg.nd, cfg.L)), cfg.io), device)
    w = to_dev((0.5 * rng.standard_normal((cfg.nd, K))).astype(np.float32), device)
    b = to_dev((0.1 * rng.standard_normal(cfg.nd)).astype(np.float32), device)
    es = W.io_itemsize(cfg.io)
    nbytes = 2 * cfg.nb * cfg.nd * cfg.L * es + cfg.nd * (K + 1) * 4
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
            "kernel_sha": kernel_hash()}


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
    return {"metric": "backward selective-scan Gelem-steps/s (B·L·D·N), 1 GPU",
            "value": cfg.element_steps / (ms * 1e-3) / 1e9, "unit": "Gelem-steps/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": cfg.io, "data": "synthetic (seeded numpy PCG64)",
            "config": {"workload": "backward of " + cfg.name, "batch": cfg.nb, "dim": cfg.nd, "seqlen": cfg.L,
                       "dstate": cfg.N},
            "kernel_sha": kernel_hash()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mamba130m",
                    choices=sorted(WORKLOADS) + ["decode"] + sorted(CONV_WORKLOADS) + sorted(BWD_WORKLOADS))
    ap.add_argument("--hot", action="store_true", help="reuse one input copy (cache-resident)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--zoh", action="store_true", help="scan with the exact zero-order-hold input gain")
    ap.add_argument("--no-rotating", action="store_true", help="decode: skip the leg that rotates over 8 states")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a %d MiB plain copy (for scaling HBM counters)" % (COPY_CALIBRATION_BYTES >> 20))
    args = ap.parse_args()
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
    if args.workload == "decode":
        res = bench_decode(args, device)
    elif args.workload in CONV_WORKLOADS:
        res = bench_conv(args, device)
    elif args.workload in BWD_WORKLOADS:
        res = bench_bwd(args, device)
    else:
        res = bench_scan(args, device)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
