#!/usr/bin/env python3
"""Decode-step benchmark of the VBQ fused dequantize-and-multiply GEMVs on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode9b]

One step = every GEMV of one synthetic decoder step (stage order qkv, o, gate,
up, down per layer, then the LM head), M = 1, weights packed in VBQ1 and
resident in HBM before timing.  Prints ONE JSON line with us/step, the
achieved algorithmic HBM bandwidth of the GEMV kernel (HIP events around every
launch, on the launch stream), the on-GPU fp16 dense control and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12  # MI355X HBM3E, bytes/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode9b", choices=["decode9b", "decode1b", "mlp1b", "linear768"])
    ap.add_argument("--mode", default="graph", choices=["graph", "eager"], help="how the step is launched")
    ap.add_argument("--no-control", action="store_true", help="skip the fp16 dense control")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU work budget of the baseline sample")
    ap.add_argument("--kernel-steps", type=int, default=5, help="steps timed with per-launch events")
    return ap.parse_args(argv)


def time_steps(torch, fn, steps):
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps  # ms per step


def sleep_cycles(torch, seconds):
    """Device-clock cycles of torch's bounded sleep kernel that last about `seconds`."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cyc = 1_000_000
    torch.cuda._sleep(cyc)  # warm up
    torch.cuda.synchronize()
    a.record()
    torch.cuda._sleep(cyc)
    b.record()
    torch.cuda.synchronize()
    per_s = cyc / max(a.elapsed_time(b) * 1e-3, 1e-6)
    return int(per_s * seconds)


def cpu_baseline(step, budget_s):
    """The oracle (plain C, one thread) on a bounded row sample of every matrix of
    the step, scaled by N / rows to a whole step."""
    import numpy as np

    import oracle
    from decode_gemv_vbq_amd import workload as wl

    W = step.W
    # calibrate: time a small slice of the largest-K matrix
    spec0 = max(W.mats, key=lambda s: s.K)
    q, b, s, x = wl.draw_matrix(spec0, W.wid, M=step.M, outliers=W.outliers, N=8)
    t0 = time.perf_counter()
    oracle.gemv(q, b, s, x)
    per_weight = (time.perf_counter() - t0) / (8 * spec0.K)
    total_weights = sum(sp.N * sp.K for sp in W.mats)
    frac = min(1.0, budget_s / max(per_weight * total_weights, 1e-9))
    est_total = 0.0
    sampled_rows = 0
    spent = 0.0
    for sp in W.mats:
        rows = max(1, int(round(sp.N * frac)))
        q, b, s, x = wl.draw_matrix(sp, W.wid, M=step.M, outliers=W.outliers, N=rows)
        t0 = time.perf_counter()
        oracle.gemv(q, b, s, x)
        dt = time.perf_counter() - t0
        spent += dt
        est_total += dt * sp.N / rows
        sampled_rows += rows
    return {
        "value": est_total * 1e6, "unit": "us/step", "cores": 1, "kind": "oracle",
        "sample": f"{sampled_rows} rows ({frac:.4f} of every matrix's rows, seeded host draw of the same "
                  f"distributions), {spent:.1f} s measured, scaled by N/rows per matrix",
    }


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import decode_gemv_vbq_amd as v
    from decode_gemv_vbq_amd import accounting as acc
    from decode_gemv_vbq_amd.step import DecodeStep

    v.lib()
    assert torch.cuda.is_available(), "bench needs a GPU"
    log(f"{v.version()} on {torch.cuda.get_device_name(0)}")
    step = DecodeStep(args.workload, M=1, log=log)
    n_launch = len(step.mats)
    alg = step.alg_bytes()
    log(f"{args.workload}: {n_launch} GEMVs, {step.weights() / 1e9:.3f} B weights, mean {step.mean_bits():.3f} bits, "
        f"{alg / 1e6:.1f} MB algorithmic, {step.layout_bytes() / 1e6:.1f} MB with row padding")

    fn = step.run
    if args.mode == "graph":
        step.capture()
        fn = step.replay
    for _ in range(args.warmup):
        fn()
    ms = time_steps(torch, fn, args.steps)
    log(f"step: {ms * 1e3:.1f} us ({args.mode}), {alg / (ms * 1e-3) / 1e9:.0f} GB/s algorithmic")

    # per-launch kernel durations: events on the launch stream around every
    # launch, all launches queued behind a bounded device sleep so they run back
    # to back (the host enqueues far slower than the GPU executes)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step.run_timed_kernels()
    torch.cuda.synchronize()
    host_s = time.perf_counter() - t0
    hold = sleep_cycles(torch, 2.0 * host_s + 0.005)
    per_kind = {}
    kern_ms = 0.0
    for _ in range(args.kernel_steps):
        ev = step.run_timed_kernels(hold_cycles=hold)
        torch.cuda.synchronize()
        for m, (a, b) in zip(step.mats, ev):
            t = a.elapsed_time(b)
            kern_ms += t
            k = per_kind.setdefault(m.spec.name, [0.0, 0, 0])
            k[0] += t
            k[1] += 1
    kern_ms /= args.kernel_steps
    for m in step.mats:
        per_kind[m.spec.name][2] += acc.vbq_read_bytes(m.L, step.M)
    kinds = {}
    for name, (t, n, bts) in per_kind.items():
        cnt = n // args.kernel_steps
        kinds[name] = {"launches": cnt, "us": round(1e3 * t / n, 2),
                       "GBps": round((bts / cnt) / (t / n * 1e-3) / 1e9, 1)}
    avg_launch_s = kern_ms * 1e-3 / n_launch
    alg_per_launch = alg / n_launch
    achieved = alg_per_launch / avg_launch_s
    log(f"kernels: {kern_ms * 1e3:.1f} us summed, {avg_launch_s * 1e6:.2f} us/launch avg, {achieved / 1e9:.0f} GB/s; "
        + ", ".join(f"{k} {d['us']} us {d['GBps']} GB/s" for k, d in kinds.items()))

    control = None
    if not args.no_control:
        step.build_control()
        cfn = step.run_control
        if args.mode == "graph":
            step.capture_control()
            cfn = step.graph16.replay
        for _ in range(max(1, args.warmup // 2)):
            cfn()
        cms = time_steps(torch, cfn, max(3, args.steps // 5))
        dense = step.dense_bytes()
        control = {"us_per_step": cms * 1e3, "GBps": dense / (cms * 1e-3) / 1e9, "bytes": dense,
                   "speedup_vbq": cms / ms}
        log(f"fp16 control: {cms * 1e3:.1f} us/step, {control['GBps']:.0f} GB/s, VBQ speedup {cms / ms:.2f}x")
        step.free_control()
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        log("CPU oracle baseline ...")
        cpu = cpu_baseline(step, args.cpu_seconds)
        log(f"CPU oracle: {cpu['value'] / 1e6:.1f} s/step (scaled), {cpu['sample']}")

    gbps = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": "us per decode step + achieved HBM GB/s (% of peak) for mixed-bit GEMV, M=1",
        "value": round(ms * 1e3, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "M": 1, "gemvs_per_step": n_launch, "launch": args.mode,
            "weights": step.weights(), "mean_bits": round(step.mean_bits(), 4),
            "alg_bytes_per_step": alg, "layout_bytes_per_step": step.layout_bytes(),
            "GBps_step": round(gbps, 1), "pct_peak_step": round(100 * gbps * 1e9 / PEAK_HBM, 2),
            "fp16_control": None if control is None else {k: round(x, 3) if isinstance(x, float) else x
                                                          for k, x in control.items()},
            "arith": "fp16 codes x fp16 activations, fp32 accumulate",
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM, 4), "traffic": None,
            "kernel": "k_gemv_wave<1> (vbq_gemv)", "alg_bytes_per_launch": round(alg_per_launch),
            "avg_launch_us": round(avg_launch_s * 1e6, 3), "per_matrix": kinds,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
