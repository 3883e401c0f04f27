#!/usr/bin/env python3
"""Decode-step benchmark of the VBQ fused dequantize-and-multiply GEMVs on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode9b]

One step = every GEMV of one synthetic decoder step (stage order qkv, o,
gate||up, down per layer, then the LM head; gate and up read the same
activations and share one launch), M = 1, weights packed in VBQ1, prepared
once into GEMV plans (the default path; --path vbq1 reads the blobs
directly) and resident in HBM before timing.  Prints ONE JSON line with us/step, the
achieved algorithmic HBM bandwidth of the GEMV kernel (per-launch duration from
HIP events around the captured step graph, on the launch stream),
the on-GPU fp16 dense control and the CPU oracle timed on a bounded sample of
the same workload.
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
PEAK_F16 = 2.5e15  # MI355X dense fp16 matrix cores, flop/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode9b", choices=["decode9b", "decode1b", "mlp1b", "linear768", "batched70b"],
                    help="decode steps (M = 1), or batched70b: the 28672x8192 up and 8192x28672 down projections "
                         "for M in {1, 4, 8, 16} tokens, clustered / uniform 4-bit / all-8-bit widths")
    ap.add_argument("--mode", default="graph", choices=["graph", "eager"], help="how the step is launched")
    ap.add_argument("--path", default="plan", choices=["plan", "vbq1"],
                    help="GEMVs from prepared plans (default) or straight from the VBQ1 blobs")
    ap.add_argument("--no-control", action="store_true", help="skip the fp16 dense control")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU work budget of the baseline: each of its single-thread runs takes about a quarter")
    ap.add_argument("--kernel-steps", type=int, default=5, help="replays of each per-kind kernel graph")
    ap.add_argument("--no-kinds", action="store_true",
                    help="skip the per-kind kernel timing (profiles then see only the step's own launches)")
    ap.add_argument("--op", default="step", choices=["step", "quantize", "argmax", "swiglu", "prefill"],
                    help="step: the decode step (the headline line); quantize: vbq_quantize of the 9B gate "
                         "projection's fp16 weights (14336x4096) with its width mix; argmax: the 9B LM head "
                         "(128256x4096) as vbq_gemv_planned_argmax against vbq_gemv_planned with fp16 logits; swiglu: "
                         "the 9B gate and up projections as one interleaved matrix with the SwiGLU epilogue "
                         "against the shared two-output launch; prefill: vbq_gemm (M > 16 tokens on the "
                         "matrix cores) on the 28672x8192 up and 8192x28672 down projections of the batched "
                         "workload against the fp16 GEMM of the dequantized weights")
    ap.add_argument("--prefill-m", default="32,64,128,256,512,2048",
                    help="token counts of the prefill sweep (the JSON line reports the one --prefill-head names)")
    ap.add_argument("--prefill-head", type=int, default=256, help="token count the prefill line reports")
    ap.add_argument("--batched-m", default="1,4,8,16,32", help="token counts of the batched workload")
    ap.add_argument("--variants", default="clustered,u4,u8", help="width variants of the batched workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 5 times (scales HBM counters) and exit")
    return ap.parse_args(argv)


def step_percentiles(torch, fn, steps):
    """Per-step durations (events between consecutive steps on the launch
    stream): median, p10 and p90 in us."""
    import numpy as np
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    d = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps)])
    return {"median": round(float(np.median(d)), 2), "p10": round(float(np.percentile(d, 10)), 2),
            "p90": round(float(np.percentile(d, 90)), 2)}


def time_steps(torch, fn, steps):
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps  # ms per step


KERNELS = {  # path -> (kernel, entry point, profile name, sources)
    "plan": ("k_gemv_plan1<KP> / k_gemv_plan2<KP> (the k_gemv_plan body, one token, preloaded arguments)",
             "vbq_gemv_planned", "k_gemv_plan", ("vbq_plan.hip", "vbq_unpack.h", "vbq_common.h")),
    "vbq1": ("k_gemv_stream<1>", "vbq_gemv", "k_gemv_stream", ("vbq_stream.hip", "vbq_unpack.h", "vbq_common.h")),
    "mfma": ("k_gemv_mfma", "vbq_gemv_batched", "k_gemv_mfma", ("vbq_mfma.hip", "vbq_unpack.h", "vbq_common.h")),
}


def kernel_source_hash(path="plan"):
    import hashlib
    h = hashlib.sha256()
    for f in KERNELS[path][3]:
        with open(os.path.join(ROOT, "decode_gemv_vbq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kpath="plan"):
    """HBM bytes per launch of the GEMV kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE x its copy-calibrated factor + WRITE_SIZE), or None when the
    kernel source has changed since the counters were taken."""
    t = profile_json(workload, kpath, "traffic")
    if t is None:
        return None
    return round(t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"])


def profile_json(workload, kpath, key):
    """The `key-json:` line of profiles/<kernel>_<workload>.md, or None when it
    is missing or the kernel source has changed since it was measured."""
    path = os.path.join(ROOT, "profiles", f"{KERNELS[kpath][2]}_{workload}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith(key + "-json: "):
            t = json.loads(line[len(key) + 7:])
            return t if t.get("kernel_source_sha") == kernel_source_hash(kpath) else None
    return None


def cpu_info():
    """(CPU model string, host threads this process may run on, capped at 16)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, max(1, min(avail, 16))


def oracle_rate():
    """Seconds per weight of the oracle GEMV (one thread, M = 1), measured on a
    small host draw: sizes the CPU baseline's row sample before the step is built."""
    import oracle
    from decode_gemv_vbq_amd import workload as wl
    spec = wl.MatrixSpec("calib", 16, 4096, wl.MIX_BASE)
    q, b, s, x = wl.draw_matrix(spec, 99, M=1)
    oracle.gemv(q, b, s, x)
    t0 = time.perf_counter()
    oracle.gemv(q, b, s, x)
    return (time.perf_counter() - t0) / (16 * 4096)


def cold_copies(W) -> int:
    """Copies of workload W that a timed step runs in turn: 1 when its weights
    (estimated from the width mix) exceed the 256 MB memory-side cache, else
    enough fresh copies to stream at least 512 MB per step, so that every GEMV
    reads its weights from HBM as it would between other layers."""
    alg_one = sum(sp.N * sp.K * sum(b * f for b, f in sp.mix.items()) / 8 + sp.N * sp.G * 2 for sp in W.mats)
    return 1 if alg_one >= 256e6 else int(-(-512e6 // alg_one))


def cpu_baseline(step, reps=3, copies=1):
    """The oracle (plain C, fp64) timed on the host on the step's sampled rows:
    the same device draws the GPU multiplies, copied back when the step was
    built.  One thread, then every host thread (the sampled rows of each matrix
    split into slices run by a thread pool; ctypes releases the GIL, the oracle
    itself is unchanged), median of `reps` each, scaled by the step's weights
    over the sampled weights (per copy when the step holds `copies` copies of
    the workload)."""
    import concurrent.futures

    import numpy as np

    import oracle
    model, threads = cpu_info()
    mats = [m for m in step.mats if m.sample is not None]
    sampled = sum(m.sample[0].shape[0] * m.spec.K for m in mats)
    total = step.weights()

    def run(nthr):
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(nthr) as ex:
            futs = []
            for m in mats:
                q, bits, sc, x = m.sample
                for sl in np.array_split(np.arange(q.shape[0]), min(nthr, q.shape[0])):
                    futs.append(ex.submit(oracle.gemv, q[sl], bits[sl], sc[sl], x))
            for f in futs:
                f.result()
        return time.perf_counter() - t0

    one = sorted(run(1) for _ in range(reps))[reps // 2]
    many = sorted(run(threads) for _ in range(reps))[reps // 2]
    scale = total / sampled / copies
    return {
        "value": round(many * scale * 1e6, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
        "single_thread_us_per_step": round(one * scale * 1e6, 1), "cpu_model": model,
        "sample": f"{sum(m.sample[0].shape[0] for m in mats)} rows of the step's own device draws "
                  f"({sampled / total:.4f} of its weights), median of {reps} runs: {one:.2f} s on 1 thread, "
                  f"{many:.2f} s on {threads} threads, scaled by weights / sampled weights",
    }


PEAK_VALU = 256 * 64 * 2.4e9  # MI355X lane-instructions/s: 256 CUs x 64 lanes per clock x 2.4 GHz


def valu_lane_instr(weights, M):
    """Estimated VALU lane-instructions of a mixed-bit GEMV over `weights` for M
    tokens: about 1.2 per weight for the unpack and bookkeeping, M / 2 dot2 per
    weight (two products each) and M / 8 for the per-group epilogue."""
    return weights * (1.2 + M / 2 + M / 8)


def bench_batched(torch, v, args):
    """The batched decode workload: the 28672x8192 up and 8192x28672 down
    projections for M in {1, 4, 8, 16} tokens (and 32, which only the blob path
    and torch.matmul take) (1% outlier channels), width variants clustered (runs
    of 8 groups from the base mix), uniform 4-bit and all-8-bit.  Per (variant,
    M), one up+down pair through the prepared plans (vbq_gemv_planned: plans made
    for one-token launches at M = 1, for token pairs otherwise) and straight
    from the blobs (vbq_gemv_batched), with
    enough weight copies in turn that a round streams at least 1 GB (so each
    call reads from HBM), replayed from a HIP graph; the hand-written dense fp16
    GEMV and torch.matmul on the dequantized weights of one copy at the same
    shapes.  Rooflines: HBM (algorithmic bytes at 8 TB/s) and VALU (estimated
    lane instructions at 39.3 T/s); the larger bounds."""
    import numpy as np

    from decode_gemv_vbq_amd import accounting as acc
    from decode_gemv_vbq_amd import workload as wl
    Ms = tuple(int(m) for m in args.batched_m.split(","))
    mf_valu = profile_json("batched70b", "mfma", "valu")
    rows = []
    for variant in args.variants.split(","):
        W = wl.workload("batched70b", variant=variant)
        copies = []
        alg1 = None
        c = 0
        while True:
            pair = []
            for spec in W.mats:
                sp = wl.MatrixSpec(spec.name, spec.N, spec.K, spec.mix, c, spec.proj_id, spec.cluster)
                q, bits, sc, _ = wl.draw_matrix_torch(sp, W.wid, 1)
                blob, L = v.pack(q, bits, sc.view(torch.float16))
                del q, bits, sc
                plan, P = v.prepare(L, blob, M=2)
                plan1, P1 = v.prepare(L, blob, M=1) if 1 in Ms else (None, None)  # one-token launches
                pair.append({"spec": spec, "L": L, "blob": blob, "plan": plan, "P": P, "plan1": plan1, "P1": P1,
                             "ws": v.workspace(L, max(Ms))})
            copies.append(pair)
            alg1 = sum(acc.vbq_read_bytes(m["L"], 0) for m in pair)
            c += 1
            if c * alg1 >= 1e9:
                break
        torch.cuda.synchronize()
        weights = sum(m["spec"].N * m["spec"].K for m in copies[0])
        xs_host = {spec.K: wl.draw_x(spec, W.wid, max(16, max(Ms)), outliers=W.outliers) for spec in W.mats}
        xs = {K: torch.from_numpy(xh.view(np.int16)).cuda().view(torch.float16) for K, xh in xs_host.items()}
        w16 = [v.dequant(m["L"], m["blob"], torch.float16) for m in copies[0]]
        log(f"batched70b {variant}: {len(copies)} copies of up+down ({alg1 / 1e6:.1f} MB algorithmic each)")
        for M in Ms:
            outs = [[torch.empty((M, m["spec"].N), dtype=torch.float16, device="cuda") for m in pair]
                    for pair in copies]
            xm = {K: xv[:M] for K, xv in xs.items()}

            def planned():
                for pair, o in zip(copies, outs):
                    for m, y in zip(pair, o):
                        if M == 1:  # the plan made for one-token launches
                            v.gemv_planned(m["P1"], m["plan1"], xm[m["spec"].K], out=y)
                        else:
                            v.gemv_planned(m["P"], m["plan"], xm[m["spec"].K], out=y)

            def blobs():
                for pair, o in zip(copies, outs):
                    for m, y in zip(pair, o):
                        v.gemv_batched(m["L"], m["blob"], xm[m["spec"].K], out=y, ws=m["ws"])

            def dense():
                for m, w, y in zip(copies[0], w16, outs[0]):
                    v.dense_f16_gemv(w, xm[m["spec"].K], out=y)

            def tmm():
                for m, w, y in zip(copies[0], w16, outs[0]):
                    torch.mm(xm[m["spec"].K], w.t(), out=y)

            res = {}
            for name, fn, n in (("planned", planned, len(copies)), ("vbq_gemv_batched", blobs, len(copies)),
                                ("dense_f16", dense, 1), ("torch_matmul", tmm, 1)):
                if M > 16 and name in ("planned", "dense_f16"):  # these take at most 16 tokens
                    res[name] = float("inf")
                    continue
                fn()
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    fn()
                for _ in range(2):
                    g.replay()
                res[name] = time_steps(torch, g.replay, max(3, args.steps // 10)) / n * 1e3  # us per pair
                del g
            alg = sum(acc.vbq_read_bytes(m["L"], M) for m in copies[0])
            t_hbm = alg / PEAK_HBM
            best = min(res["planned"], res["vbq_gemv_batched"])
            mf = M >= 3 and res["vbq_gemv_batched"] <= res["planned"]
            if mf:  # the matrix-core kernel: lane instructions per weight measured by counters (at 16 tokens)
                lipw = (mf_valu or {}).get("lane_instr_per_weight", {}).get(variant)
                lane = None if lipw is None or M > 16 else lipw * weights
            else:
                lane = valu_lane_instr(weights, M)
            t_valu = None if lane is None else lane / PEAK_VALU
            row = {"variant": variant, "M": M,
                   **{f"{k}_us": None if t == float("inf") else round(t, 2) for k, t in res.items()},
                   "alg_bytes": alg, "GBps": round(alg / (best * 1e-6) / 1e9, 1),
                   "kernel": "k_gemv_mfma" if mf else "k_gemv_plan",
                   "valu_lane_instr": lane,
                   "hbm_frac": round(t_hbm / (best * 1e-6), 4),
                   "valu_frac": None if t_valu is None else round(t_valu / (best * 1e-6), 4),
                   "bound": "hbm" if t_valu is None or t_valu <= t_hbm else "alu",
                   "speedup_vs_dense_f16": None if res["dense_f16"] == float("inf") else round(res["dense_f16"] / best, 3),
                   "speedup_vs_torch_matmul": round(res["torch_matmul"] / best, 3)}
            rows.append(row)
            log((f"  M={M:2d}: planned {res['planned']:.1f} us, vbq_gemv_batched {res['vbq_gemv_batched']:.1f} us, "
                 f"dense fp16 {res['dense_f16']:.1f} us, torch.matmul {res['torch_matmul']:.1f} us; ").replace("inf us", "n/a")
                + f"{row['GBps']} GB/s, {100 * row['hbm_frac']:.1f}% of HBM, "
                + ("VALU model unmeasured" if row["valu_frac"] is None else f"{100 * row['valu_frac']:.1f}% of VALU")
                + f" ({row['kernel']})")
            del outs
        del copies, w16, xs
        torch.cuda.empty_cache()
    head = next((r for r in rows if r["variant"] == "clustered" and r["M"] == 16), rows[-1])
    t = min(head["planned_us"], head["vbq_gemv_batched_us"]) * 1e-6
    mf = head["kernel"] == "k_gemv_mfma"
    if head["bound"] == "alu":
        ach = head["valu_lane_instr"] / t
        roof = {"bound": "alu", "achieved": round(ach / 1e12, 2), "peak": round(PEAK_VALU / 1e12, 2),
                "unit": "T lane-instr/s", "frac": round(ach / PEAK_VALU, 4)}
    else:
        roof = {"bound": "hbm", "achieved": head["GBps"], "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": head["hbm_frac"]}
    roof.update({"traffic": None,
                 "kernel": ("k_gemv_mfma (vbq_gemv_batched, 64-row workgroups, K split when the workspace allows)"
                            if mf else "k_gemv_plan<2, 0> (vbq_gemv_planned, launches of 2 tokens)"),
                 "valu_model": ("lane instructions per weight from the committed SQ_INSTS_VALU counters"
                                if mf else "1.2 + M/2 + M/8 lane instructions per weight")})
    print(json.dumps({
        "metric": "us per batched decode up+down GEMV pair (28672x8192 + 8192x28672, M=16 tokens)",
        "value": min(head["planned_us"], head["vbq_gemv_batched_us"]), "unit": "us", "n_gpus": 1,
        "steps": max(3, args.steps // 10), "warmup": 2, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "batched70b: up 28672x8192 + down 8192x28672, M in {1,4,8,16}, clustered / u4 / u8 "
                               "widths, 1% outlier channels; weight copies in turn, >= 1 GB per round",
                   "M": 16, "variant": "clustered", "sweep": rows},
        "roofline": roof, "cpu_baseline": None}), flush=True)


def bench_quantize(torch, v, args):
    """vbq_quantize on a 14336x4096 fp16 weight matrix with the 9B model's width
    mix; bytes are the weights read, the widths read, the codes and scales
    written (an HBM-bound elementwise pass)."""
    from decode_gemv_vbq_amd import workload as wl
    N, K = 14336, 4096
    G = K // 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260703)
    w = torch.randn((N, K), generator=gen, device="cuda", dtype=torch.float32).half()
    widths = sorted(wl.MIX_BASE)
    p = torch.tensor([wl.MIX_BASE[b] for b in widths], dtype=torch.float32, device="cuda")
    idx = torch.multinomial(p, N * G, replacement=True, generator=gen).view(N, G)
    bits = torch.tensor(widths, dtype=torch.uint8, device="cuda")[idx].contiguous()
    for _ in range(3):
        v.quantize(w, bits)
    reps = max(5, args.steps // 2)
    q = s = None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        q, s = v.quantize(w, bits)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * N * K + N * G + N * K + 2 * N * G
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"vbq_quantize {N}x{K} fp16: {ms * 1e3:.1f} us, {gbps:.0f} GB/s")
    print(json.dumps({
        "metric": "us per vbq_quantize call (fp16 weights -> codes + fp16 scales)", "value": round(ms * 1e3, 2),
        "unit": "us", "n_gpus": 1, "steps": reps, "warmup": 3, "higher_is_better": False, "dtype": "f32",
        "data": "synthetic", "config": {"workload": "quantize 14336x4096 fp16, 9B width mix", "bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(gbps * 1e9 / PEAK_HBM, 4), "traffic": None, "kernel": "k_quantize (vbq_quantize)"},
        "cpu_baseline": None}), flush=True)


def bench_swiglu(torch, v, args):
    """The 9B MLP's gate and up projections (2 x 14336x4096) for one token:
    one interleaved 28672-row matrix with the SwiGLU epilogue (14336 outputs)
    against the step's shared launch of the two matrices (two 14336-row
    outputs).  Ten copies are used in turn so each call streams from HBM."""
    from decode_gemv_vbq_amd import workload as wl
    from decode_gemv_vbq_amd import accounting as acc
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    copies = []
    for c in range(10):
        g = wl.draw_matrix_torch(wl.MatrixSpec("gate", 14336, 4096, wl.MIX_BASE, layer=c), 97, 1)
        u = wl.draw_matrix_torch(wl.MatrixSpec("up", 14336, 4096, wl.MIX_BASE, layer=c), 98, 1)
        x = g[3]
        qi = torch.stack((g[0], u[0]), 1).view(28672, 4096)
        bi = torch.stack((g[1], u[1]), 1).view(28672, 64)
        si = torch.stack((g[2], u[2]), 1).view(28672, 64)
        blob_i, L_i = v.pack(qi, bi, si.view(torch.float16))
        plan_i, P_i = v.prepare(L_i, blob_i, M=1)
        sep = []
        for t in (g, u):
            blob, L = v.pack(t[0], t[1], t[2].view(torch.float16))
            plan, P = v.prepare(L, blob, M=1, wgs=cus // 2)
            sep.append((P, plan, L, blob))
        del qi, bi, si, g, u
        copies.append({"x": x, "P": P_i, "plan": plan_i, "L": L_i, "blob": blob_i, "sep": sep,
                       "h": torch.empty((1, 14336), dtype=torch.float16, device="cuda"),
                       "yg": torch.empty((1, 14336), dtype=torch.float16, device="cuda"),
                       "yu": torch.empty((1, 14336), dtype=torch.float16, device="cuda")})
    torch.cuda.synchronize()

    def run_swiglu():
        for c in copies:
            v.gemv_planned_swiglu(c["P"], c["plan"], c["x"], out=c["h"])

    def run_shared():
        for c in copies:
            v.gemv_planned_shared([(P, plan) for P, plan, _, _ in c["sep"]], c["x"], outs=[c["yg"], c["yu"]])

    res = {}
    for name, fn in (("swiglu", run_swiglu), ("shared", run_shared)):
        fn()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        for _ in range(2):
            gr.replay()
        res[name] = time_steps(torch, gr.replay, max(5, args.steps // 5)) / len(copies) * 1e3
    alg = acc.vbq_read_bytes(copies[0]["L"], 1)
    gbps = alg / (res["swiglu"] * 1e-6) / 1e9
    log(f"gate+up 2x14336x4096: SwiGLU epilogue {res['swiglu']:.1f} us, shared two-output launch {res['shared']:.1f} us")
    print(json.dumps({
        "metric": "us per SwiGLU MLP-input call (gate and up GEMVs with the activation fused, M=1)",
        "value": round(res["swiglu"], 2), "unit": "us", "n_gpus": 1, "steps": max(5, args.steps // 5),
        "warmup": 2, "higher_is_better": False, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "gate+up 2x14336x4096 interleaved, base width mix, 10 copies in turn",
                   "shared_two_output_us": round(res["shared"], 2), "alg_bytes": alg},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(gbps * 1e9 / PEAK_HBM, 4), "traffic": None,
                     "kernel": "k_gemv_plan1<2, KP> SwiGLU epilogue, preloaded arguments (vbq_gemv_planned_swiglu)"},
        "cpu_baseline": None}), flush=True)


def bench_argmax(torch, v, args):
    """The 9B LM head (128256x4096, head width mix) for one token: greedy
    argmax epilogue (no logits written) against the plain planned GEMV writing
    fp16 logits.  Three copies of the matrix are used in turn so that each call
    streams its weights from HBM (the three exceed the memory-side cache)."""
    from decode_gemv_vbq_amd import workload as wl
    from decode_gemv_vbq_amd import accounting as acc
    spec = wl.MatrixSpec("head", 128256, 4096, wl.MIX_HEAD, layer=0)
    mats = []
    for c in range(3):
        q, bits, s, x = wl.draw_matrix_torch(spec, 94 + c, 1)
        blob, L = v.pack(q, bits, s.view(torch.float16))
        del q, bits, s
        plan, P = v.prepare(L, blob, M=1)
        mats.append((L, blob, plan, P, x))
    torch.cuda.synchronize()
    ws = v.argmax_workspace()
    ys = [torch.empty((1, spec.N), dtype=torch.float16, device="cuda") for _ in mats]

    def run_argmax():
        for L, blob, plan, P, x in mats:
            v.gemv_planned_argmax(P, plan, x, ws=ws)

    def run_logits():
        for (L, blob, plan, P, x), y in zip(mats, ys):
            v.gemv_planned(P, plan, x, out=y)

    res = {}
    for name, fn in (("argmax", run_argmax), ("logits", run_logits)):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(3):
            g.replay()
        res[name] = time_steps(torch, g.replay, max(10, args.steps // 2)) / len(mats) * 1e3  # us per call
    alg = acc.vbq_read_bytes(mats[0][0], 1)
    gbps = alg / (res["argmax"] * 1e-6) / 1e9
    log(f"LM head 128256x4096: argmax {res['argmax']:.1f} us, logits {res['logits']:.1f} us per call")
    print(json.dumps({
        "metric": "us per greedy-decode LM-head call (argmax epilogue, M=1)", "value": round(res["argmax"], 2),
        "unit": "us", "n_gpus": 1, "steps": max(10, args.steps // 2), "warmup": 3, "higher_is_better": False,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "LM head 128256x4096, head width mix, 3 copies in turn",
                   "logits_us": round(res["logits"], 2), "alg_bytes": alg},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(gbps * 1e9 / PEAK_HBM, 4), "traffic": None,
                     "kernel": "k_gemv_plan<1, 1> argmax epilogue (vbq_gemv_planned_argmax)"},
        "cpu_baseline": None}), flush=True)


def bench_prefill(torch, v, args):
    """Prefill GEMMs: the batched workload's 28672x8192 up and 8192x28672 down
    projections (clustered widths, 1% outlier channels) for M tokens, as
    vbq_gemm from GEMM plans against torch's fp16 GEMM (hipBLASLt) of the
    dequantized weights, and for up to 32 tokens vbq_gemv_batched straight from
    the blobs (the matrix-core GEMV).  Two copies of each matrix are used in turn so that
    each call streams its weights from HBM; every path is replayed from a HIP
    graph.  Roofline per M: the larger of the plan bytes at 8 TB/s and
    2 M N K flops at the dense fp16 matrix-core peak."""
    from decode_gemv_vbq_amd import workload as wl
    from decode_gemv_vbq_amd import accounting as acc
    wk = wl.workload("batched70b")
    ms = sorted({int(m) for m in args.prefill_m.split(",")} | {args.prefill_head})
    mats = []
    for c in range(2):
        for spec in wk.mats:
            q, bits, s, _ = wl.draw_matrix_torch(wl.MatrixSpec(spec.name, spec.N, spec.K, spec.mix, c, spec.proj_id,
                                                               spec.cluster), wk.wid, 1)
            blob, L = v.pack(q, bits, s.view(torch.float16))
            del q, bits, s
            buf, GP = v.gemm_prepare(L, blob)
            w16 = v.dequant(L, blob, torch.float16)
            mats.append({"spec": spec, "L": L, "buf": buf, "GP": GP, "w16": w16, "blob": blob,
                         "ws_b": v.workspace(L, 32)})
    torch.cuda.synchronize()
    plan_bytes = sum(m["GP"].total_bytes for m in mats[:2])
    alg_w = sum(acc.vbq_read_bytes(m["L"], 0) for m in mats[:2])
    log(f"GEMM plans: {plan_bytes / 1e6:.1f} MB for up+down ({alg_w / 1e6:.1f} MB packed), "
        f"slots {[m['GP'].slot_bytes for m in mats[:2]]}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    rows = []
    for M in ms:
        xs = {K: (torch.randn((M, K), generator=gen, device="cuda", dtype=torch.float32)).half()
              for K in {m["spec"].K for m in mats}}
        ws = v.gemm_workspace(mats[0]["GP"], M)
        ws2 = v.gemm_workspace(mats[1]["GP"], M)
        wsz = ws if ws.numel() >= ws2.numel() else ws2
        outs = [torch.empty((M, m["spec"].N), dtype=torch.float16, device="cuda") for m in mats]

        def run_vbq():
            for m, o in zip(mats, outs):
                v.gemm(m["GP"], m["buf"], xs[m["spec"].K], out=o, ws=wsz)

        def run_f16():
            for m, o in zip(mats, outs):
                torch.mm(xs[m["spec"].K], m["w16"].t(), out=o)

        def run_batched():  # up to 32 tokens: the matrix-core GEMV straight from the blobs
            for m, o in zip(mats, outs):
                v.gemv_batched(m["L"], m["blob"], xs[m["spec"].K], out=o, ws=m["ws_b"])

        res = {}
        paths = (("vbq", run_vbq), ("f16", run_f16)) + ((("batched", run_batched),) if M <= 32 else ())
        for name, fn in paths:
            fn()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                fn()
            for _ in range(2):
                gr.replay()
            res[name] = time_steps(torch, gr.replay, max(5, args.steps // 5)) / (len(mats) // 2) * 1e3
        flops = sum(2.0 * M * m["spec"].N * m["spec"].K for m in mats[:2])
        byts = alg_w + sum(2 * M * m["spec"].K + 2 * M * m["spec"].N for m in mats[:2])
        t_mfma, t_hbm = flops / PEAK_F16, byts / PEAK_HBM
        bound = "mfma" if t_mfma >= t_hbm else "hbm"
        t = res["vbq"] * 1e-6
        row = {"M": M, "us": round(res["vbq"], 2), "f16_us": round(res["f16"], 2),
               "speedup_vs_f16": round(res["f16"] / res["vbq"], 3), "bound": bound,
               "vbq_gemv_batched_us": round(res["batched"], 2) if "batched" in res else None,
               "speedup_batched_vs_f16": round(res["f16"] / res["batched"], 3) if "batched" in res else None,
               "TFLOPs": round(flops / t / 1e12, 1), "GBps": round(byts / t / 1e9, 1),
               "frac": round(max(t_mfma, t_hbm) / t, 4)}
        rows.append(row)
        log(f"M={M}: vbq_gemm {res['vbq']:.1f} us ({row['TFLOPs']} TFLOP/s, {row['GBps']} GB/s, "
            f"{100 * row['frac']:.1f}% of the {bound} roof), fp16 GEMM {res['f16']:.1f} us, "
            f"speedup {row['speedup_vs_f16']:.2f}x"
            + (f"; vbq_gemv_batched {res['batched']:.1f} us ({row['speedup_batched_vs_f16']:.2f}x)" if "batched" in res
               else ""))
        del xs, ws, ws2, wsz, outs
    head = next(r for r in rows if r["M"] == args.prefill_head)
    if head["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": head["TFLOPs"], "peak": PEAK_F16 / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": head["GBps"], "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof.update({"frac": round(roof["achieved"] / roof["peak"], 4), "traffic": None,
                 "kernel": "k_xpair + k_gemm<MT> (vbq_gemm), whole calls"})
    print(json.dumps({
        "metric": f"us per prefill up+down GEMM pair (M={args.prefill_head} tokens)",
        "value": head["us"], "unit": "us", "n_gpus": 1, "steps": max(5, args.steps // 5), "warmup": 2,
        "higher_is_better": False, "dtype": "f16 x f16 -> f32 (matrix cores)", "data": "synthetic",
        "vs_baseline": None,
        "config": {"workload": "batched70b up 28672x8192 + down 8192x28672, clustered widths, M tokens",
                   "M": args.prefill_head, "fp16_gemm_us": head["f16_us"], "speedup_vs_f16": head["speedup_vs_f16"],
                   "plan_bytes": plan_bytes, "sweep": rows},
        "roofline": roof, "cpu_baseline": None}), flush=True)


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel(), "copy_bytes_written": dst.numel(), "copies": 5}))
        return

    import decode_gemv_vbq_amd as v
    from decode_gemv_vbq_amd import accounting as acc
    from decode_gemv_vbq_amd.step import DecodeStep

    if args.op == "quantize":
        bench_quantize(torch, v, args)
        return
    if args.op == "argmax":
        bench_argmax(torch, v, args)
        return
    if args.op == "swiglu":
        bench_swiglu(torch, v, args)
        return
    if args.op == "prefill":
        bench_prefill(torch, v, args)
        return

    v.lib()
    assert torch.cuda.is_available(), "bench needs a GPU"
    log(f"{v.version()} on {torch.cuda.get_device_name(0)}")
    if args.workload == "batched70b":
        bench_batched(torch, v, args)
        return
    from decode_gemv_vbq_amd import workload as wl
    one = wl.workload(args.workload)
    copies = cold_copies(one)
    frac = 0.0
    if not args.no_cpu:
        # the CPU baseline's row sample: about cpu_seconds / 4 per single-thread run
        total_w = sum(sp.N * sp.K for sp in one.mats)  # rows are sampled from the first copy
        frac = min(1.0, args.cpu_seconds / 4 / (oracle_rate() * total_w))
    step = DecodeStep(args.workload, M=1, log=log, planned=args.path == "plan", sample_frac=frac, copies=copies)
    n_launch = len(step.stages)
    alg = step.alg_bytes()
    if copies > 1:
        log(f"{copies} copies of the workload in turn ({alg / 1e6:.0f} MB per round); the JSON figures are per copy")
    log(f"{args.workload}: {len(step.mats)} GEMVs in {n_launch} launches, {step.weights() / 1e9:.3f} B weights, mean {step.mean_bits():.3f} bits, "
        f"{alg / 1e6:.1f} MB algorithmic, {step.layout_bytes() / 1e6:.1f} MB with row padding")

    fn = step.run
    if args.mode == "graph":
        step.capture()
        fn = step.replay
    for _ in range(args.warmup):
        fn()
    ms = time_steps(torch, fn, args.steps)
    dist = step_percentiles(torch, fn, args.steps)
    log(f"step: {ms * 1e3:.1f} us ({args.mode}), {alg / (ms * 1e-3) / 1e9:.0f} GB/s algorithmic; per step "
        f"median {dist['median']} us, p10 {dist['p10']}, p90 {dist['p90']}")

    # per-launch kernel durations: for each stage kind, that kind's launches of
    # one step captured back to back in a graph (events on the launch stream);
    # a kind with fewer than 8 launches per step (the LM head) is repeated to 8
    # in its graph, so that the graph's own launch cost is spread as for the others
    kinds = {}
    kern_ms = 0.0
    names = []
    for st in step.stages:
        if step.stage_name(st) not in names:
            names.append(step.stage_name(st))
    for name in ([] if args.no_kinds else names):
        sts = [st for st in step.stages if step.stage_name(st) == name]
        rep_in = -(-8 // len(sts))
        g = step.capture_stages(sts * rep_in)
        for _ in range(2):
            g.replay()
        reps = max(2, args.kernel_steps)
        t = time_steps(torch, g.replay, reps) / (len(sts) * rep_in)  # ms per launch
        del g
        bts = sum(acc.vbq_read_bytes(step.mats[i].L, step.M) for st in sts for i in st) / len(sts)
        kinds[name] = {"launches": len(sts) // copies, "us": round(t * 1e3, 2), "GBps": round(bts / (t * 1e-3) / 1e9, 1)}
        kern_ms += t * len(sts)
    # the roofline uses the cold step: its launches run back to back in the graph,
    # so the average launch duration is the step time over the launch count
    avg_launch_s = ms * 1e-3 / n_launch
    alg_per_launch = alg / n_launch
    achieved = alg_per_launch / avg_launch_s
    log(f"kernels: {avg_launch_s * 1e6:.2f} us/launch avg in the step, {achieved / 1e9:.0f} GB/s; per kind (replayed "
        f"alone, {kern_ms * 1e3:.1f} us summed): " + ", ".join(f"{k} {d['us']} us {d['GBps']} GB/s" for k, d in kinds.items()))
    traffic = measured_traffic(args.workload, args.path)

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
        control = {"us_per_step": cms * 1e3 / copies, "GBps": dense / (cms * 1e-3) / 1e9, "bytes": dense // copies,
                   "speedup_vbq": cms / ms}
        log(f"fp16 control: {cms * 1e3:.1f} us/step, {control['GBps']:.0f} GB/s, VBQ speedup {cms / ms:.2f}x")
        # the library's fp16 GEMV (torch.matmul: rocBLAS / hipBLASLt) at the same shapes
        tfn = step.run_torch_control
        if args.mode == "graph":
            tfn = step.capture_torch_control().replay
        for _ in range(max(1, args.warmup // 2)):
            tfn()
        tms = time_steps(torch, tfn, max(3, args.steps // 5))
        control.update({"torch_matmul_us_per_step": tms * 1e3 / copies, "torch_matmul_GBps": dense / (tms * 1e-3) / 1e9,
                        "speedup_vbq_vs_torch_matmul": tms / ms})
        log(f"torch.matmul fp16: {tms * 1e3:.1f} us/step, {dense / (tms * 1e-3) / 1e9:.0f} GB/s, "
            f"VBQ speedup {tms / ms:.2f}x")
        step.free_control()
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        log("CPU oracle baseline ...")
        cpu = cpu_baseline(step, copies=copies)
        log(f"CPU oracle: {cpu['value'] / 1e6:.2f} s/step on {cpu['cores']} threads "
            f"({cpu['single_thread_us_per_step'] / 1e6:.2f} s on one), {cpu['cpu_model']}; {cpu['sample']}")

    gbps = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": "us per decode step + achieved HBM GB/s (% of peak) for mixed-bit GEMV, M=1",
        "value": round(ms * 1e3 / copies, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / copies, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "M": 1, "gemvs_per_step": len(step.mats) // copies,
            "launches_per_step": n_launch // copies, "launch": args.mode, "path": args.path,
            "copies": copies, "copies_note": None if copies == 1 else
            f"{copies} copies of the workload (fresh draws) run in turn per timed step so that the weights stream "
            f"from HBM, not the memory-side cache; every per-step figure is the round's figure / {copies}",
            "plan_bytes_per_step": step.plan_bytes() // copies if step.planned else None,
            "weights": step.weights() // copies, "mean_bits": round(step.mean_bits(), 4),
            "alg_bytes_per_step": alg // copies, "layout_bytes_per_step": step.layout_bytes() // copies,
            "GBps_step": round(gbps, 1), "pct_peak_step": round(100 * gbps * 1e9 / PEAK_HBM, 2),
            "us_per_step_median": round(dist["median"] / copies, 2), "us_per_step_p10": round(dist["p10"] / copies, 2),
            "us_per_step_p90": round(dist["p90"] / copies, 2),
            "fp16_control": None if control is None else {k: round(x, 3) if isinstance(x, float) else x
                                                          for k, x in control.items()},
            "arith": "fp16 codes x fp16 activations, fp32 accumulate",
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM, 4), "traffic": traffic,
            "kernel": f"{KERNELS[args.path][0]} ({KERNELS[args.path][1]})", "alg_bytes_per_launch": round(alg_per_launch),
            "avg_launch_us": round(avg_launch_s * 1e6, 3), "per_matrix": kinds,
            "per_matrix_sum_us": round(kern_ms * 1e3 / copies, 1) if kinds else None,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
