#!/usr/bin/env python3
"""Benchmark of the exact-attention forward pass on one MI355X.

One step = one call of the forward pass (the whole hot path is one kernel
launch) on the headline workload B=8, H=32, N=2048, d=128, bf16, non-causal,
scale 1/sqrt(d), inputs resident in HBM.  Prints ONE JSON line on stdout.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--all] [--copy-calibration BYTES] [--backward]

Throughput is counted as 4*B*H*N^2*d FLOPs per call (halved when causal).
Timing uses HIP events recorded on the stream the kernel is launched on.
The FP8 workloads (--workload b8h32n2048d128_fp8, ...) time fa2_fwd_fp8 on
E4M3 inputs with a bf16 output, against the dense FP8 MFMA peak.

--backward times the backward pass instead (one step = one fa2_bwd call:
the D, dK/dV and dQ kernels on one stream), counted as 10*B*H*N^2*d FLOPs
(the five products S, dP, dV, dK, dQ; halved when causal), and prints its
own JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS (and % of MFMA peak) at N=2048,d=128 bf16"
FP8_METRIC = "attention fwd TFLOPS (and % of FP8 MFMA peak), E4M3 inputs, 4*B*H*N^2*d FLOPs per call"
BWD_METRIC = "attention bwd TFLOPS (and % of MFMA peak), 10*B*H*N^2*d FLOPs per call"
# MI355X dense MFMA peaks: 256 CU x 2.4 GHz x 4096 FLOP/clk (16-bit), x 8192 (FP8)
PEAK_TFLOPS = {"bf16": 2516.6, "fp16": 2516.6, "fp8": 5033.2}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "exact_attention_63_amd", "csrc")
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("fa2_fwd_kernel.hpp", "fa2_fwd_sched.hpp", "fa2_fwd_sched.inc")]
FP8_KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("fa2_fwd_kernel.hpp", "fa2_fwd_fp8.hpp",
                                                       "fa2_fwd_fp8_sched.hpp", "fa2_fwd_fp8_sched.inc")]
PROBE_LIB = os.path.join(ROOT, "bench_probe.so")


def kernel_identity(w, variant: int = 0) -> str:
    """Hash of the forward kernel sources and the tile configuration that the
    workload runs with: the counters recorded for one identity are only reused
    for exactly that kernel."""
    import exact_attention_63_amd as fa2
    h = hashlib.sha256()
    if w.dtype == "fp8":
        vi = variant or fa2.lib().fa2_fp8_default_variant(w.d, int(w.causal))
        for src in FP8_KERNEL_SOURCES:
            with open(src, "rb") as f:
                h.update(f.read())
        h.update(fa2.fp8_variant_name(vi).encode())
        h.update(f"{w.dtype}/{w.d}/{int(w.causal)}".encode())
        return h.hexdigest()[:16]
    vi = variant or fa2.default_variant(0 if w.dtype == "fp16" else 1, w.d, w.causal)
    for src in KERNEL_SOURCES:
        with open(src, "rb") as f:
            h.update(f.read())
    h.update(fa2.variant_name(vi).encode())
    h.update(f"{w.dtype}/{w.d}/{int(w.causal)}".encode())
    return h.hexdigest()[:16]


def measured_traffic(w, variant: int = 0):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    the kernel changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(w.name)
    if not ent or ent.get("kernel_identity") != kernel_identity(w, variant):
        return None
    return ent.get("hbm_bytes_per_launch")


def time_gpu(fn, steps: int, warmup: int):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall / steps * 1e3


def per_call_stats(fn, calls: int):
    """Per-call durations (ms) from one HIP event pair per call on the current
    stream, taken after the timed region (they do not enter `value`)."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return {"calls": calls, "median_ms": round(t[len(t) // 2], 5), "min_ms": round(t[0], 5),
            "p90_ms": round(t[min(len(t) - 1, int(0.9 * len(t)))], 5)}


def host_info():
    """Host cores this process may run on, the BLAS thread count and the CPU model."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return cores, blas, model


def mfma_probe(iters: int = 100000, fp8: bool = False):
    """Sustained dense bf16 (or FP8) MFMA throughput (TFLOP/s) and shader clock
    (GHz) measured now by bench_probe.so (an MFMA-only loop on every CU), or
    None when the probe is not built."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        return None
    import torch
    lib = ctypes.CDLL(PROBE_LIB)
    fn = lib.fa2_probe_mfma_fp8 if fp8 else lib.fa2_probe_mfma
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    rc = fn(iters // 4 if fp8 else iters, torch.cuda.current_stream().cuda_stream, ctypes.byref(tf),
            ctypes.byref(ghz))
    if rc != 0:
        raise RuntimeError(f"MFMA probe failed with HIP error {rc}")
    inst = "v_mfma_f32_32x32x64_f8f6f4 (E4M3)" if fp8 else "v_mfma_f32_32x32x16_bf16"
    return {"value": round(tf.value, 1), "unit": "TFLOP/s", "clock_ghz": round(ghz.value, 3),
            "what": f"bench_probe.hip: back-to-back {inst}, 2 waves per SIMD on every CU, "
                    "random operands, run right after the timed region"}


def cpu_baseline(w, budget_s: float = 20.0):
    """The fp64 CPU oracle timed on whole heads of the same workload (in order)
    until about budget_s seconds of work are done or every head is done."""
    import oracle
    from workloads import workload_inputs, workload_inputs_fp8, to_f64
    host_cores, blas, model = host_info()
    cores = min(blas, host_cores)
    if w.dtype == "fp8":
        (q8, k8, v8), desc = workload_inputs_fp8(w)

        def one_head(b, h):
            oracle.attention_fp8(q8[b, h].numpy(), k8[b, h].numpy(), v8[b, h].numpy(), *desc, w.causal, w.scale)
        what = "fp64 NumPy oracle (E4M3 decoding, then the 3-pass definition)"
    else:
        q, k, v = workload_inputs(w)

        def one_head(b, h):
            oracle.attention_3pass(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), w.causal, w.scale)
        what = "fp64 NumPy 3-pass oracle"
    nh = w.B * w.H
    heads = 0
    t0 = time.perf_counter()
    while heads < nh:
        one_head(*divmod(heads, w.H))
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops_per_head = w.flops / nh
    return {"value": round(heads * flops_per_head / dt / 1e12, 6), "unit": "TFLOPS", "cores": cores,
            "host_cores": host_cores, "blas_threads": blas, "cpu_model": model, "kind": "oracle",
            "sample": f"{heads} of {nh} heads (all {w.N} rows each) of {w.name}, {what}, "
                      f"{dt:.1f} s; TFLOPS counted like the GPU figure"}


BWD_KERNEL_SOURCE = os.path.join(ROOT, "exact_attention_63_amd", "csrc", "fa2_bwd_kernel.hpp")
API_SOURCE = os.path.join(ROOT, "exact_attention_63_amd", "csrc", "fa2_api.hip")


def bwd_identity(w) -> str:
    """Hash of the backward kernel source (without its // comments, whitespace
    collapsed), the host table that instantiates the backward kernels with
    their template arguments, the host function that picks the default
    backward configuration, and dtype/d/causal."""
    import re
    h = hashlib.sha256()
    with open(BWD_KERNEL_SOURCE) as f:
        h.update(" ".join(re.sub(r"//[^\n]*", "", f.read()).split()).encode())
    with open(API_SOURCE) as f:
        api = f.read()
    for pat in (r"constexpr void fill_bwd\(.*?\n}", r"BwdKernels make_bwd_kernels\(.*?\n}",
                r"int default_bwd_variant\(.*?\n}"):
        m = re.search(pat, api, flags=re.S)
        h.update((m.group(0) if m else "").encode())
    h.update(f"{w.dtype}/{w.d}/{int(w.causal)}".encode())
    return h.hexdigest()[:16]


def measured_traffic_bwd(w, variant: int = 0):
    """HBM bytes per backward call from committed counter runs, or None."""
    if variant != 0:
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("bwd:" + w.name)
    if not ent or ent.get("kernel_identity") != bwd_identity(w):
        return None
    return ent.get("hbm_bytes_per_call")


def cpu_baseline_bwd(w, budget_s: float = 20.0):
    """The fp64 CPU gradient oracle timed on whole heads of the same workload."""
    import oracle
    from workloads import workload_grad_output, workload_inputs, to_f64
    host_cores, blas, model = host_info()
    cores = min(blas, host_cores)
    q, k, v = workload_inputs(w)
    do = workload_grad_output(w)
    nh = w.B * w.H
    heads = 0
    t0 = time.perf_counter()
    while heads < nh:
        b, h = divmod(heads, w.H)
        oracle.attention_backward(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), to_f64(do[b, h]),
                                  w.causal, w.scale)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(heads * (w.bwd_flops / nh) / dt / 1e12, 6), "unit": "TFLOPS", "cores": cores,
            "host_cores": host_cores, "blas_threads": blas, "cpu_model": model, "kind": "oracle",
            "sample": f"{heads} of {nh} heads (all {w.N} rows each) of {w.name}, fp64 NumPy gradient "
                      f"oracle, {dt:.1f} s; TFLOPS counted like the GPU figure"}


def run_backward(w, steps, warmup, variant=0):
    import torch
    import exact_attention_63_amd as fa2
    from workloads import workload_grad_output, workload_inputs
    q, k, v = (t.cuda() for t in workload_inputs(w))
    do = workload_grad_output(w).cuda()
    o, lse = fa2.forward(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty_like(lse)

    def step():
        fa2.backward(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, variant=variant, dq=dq, dk=dk, dv=dv,
                     delta=delta)

    res = time_gpu(step, steps, warmup)
    run_backward.last_stats = per_call_stats(step, steps)
    return res


def backward_main(args, w):
    ms, wall_ms = run_backward(w, args.steps, args.warmup, args.variant)
    stats = run_backward.last_stats
    peak = PEAK_TFLOPS[w.dtype]
    tflops = w.bwd_flops / (ms * 1e-3) / 1e12
    if args.all:
        from workloads import WORKLOADS
        print(f"{'workload (backward)':36s} {'ms':>9s} {'TFLOPS':>9s} {'%peak':>7s}", file=sys.stderr)
        for other in WORKLOADS.values():
            oms, _ = run_backward(other, max(5, args.steps // 2), max(2, args.warmup // 2), args.variant)
            t = other.bwd_flops / (oms * 1e-3) / 1e12
            print(f"{other.name:36s} {oms:9.4f} {t:9.1f} {100 * t / PEAK_TFLOPS[other.dtype]:6.1f}%",
                  file=sys.stderr, flush=True)
    line = {
        "metric": BWD_METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs and dO, rounded to the dtype)",
        "config": {**w.describe(), "pass": "backward (D, dK/dV, dQ kernels)", "variant": args.variant,
                   "parallelism": "single GPU",
                   "wall_ms_per_step": round(wall_ms, 5), "per_call": stats},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": measured_traffic_bwd(w, args.variant),
            "scope": "the whole call (three kernels); per-kernel durations in the rocprofv3 summary",
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_bwd(w)
    print(json.dumps(line), flush=True)


def run_workload(w, steps, warmup, variant=0):
    import torch
    import exact_attention_63_amd as fa2
    from workloads import workload_inputs, workload_inputs_fp8
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")
    if w.dtype == "fp8":
        (q8, k8, v8), desc = workload_inputs_fp8(w)
        q, k, v = (t.cuda() for t in (q8, k8, v8))
        o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")

        def step():
            fa2.forward_fp8(q, k, v, *desc, causal=w.causal, scale=w.scale, out=o, lse=lse, variant=variant)
    else:
        q, k, v = (t.cuda() for t in workload_inputs(w))
        o = torch.empty_like(q)

        def step():
            fa2.forward(q, k, v, causal=w.causal, scale=w.scale, variant=variant, out=o, lse=lse)

    ms, wall_ms = time_gpu(step, steps, warmup)
    run_workload.last_stats = per_call_stats(step, steps)
    return ms, wall_ms


def copy_calibration(nbytes: int, steps: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": steps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--variant", type=int, default=0,
                    help="tile variant of the timed pass (0 = tuned default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all", action="store_true", help="also time every workload (stderr table)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--backward", action="store_true", help="time the backward pass instead")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this forward pass is not sharded across GPUs "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return

    from workloads import FP8_WORKLOADS, HEADLINE, WORKLOADS
    name = args.workload or HEADLINE
    if name not in WORKLOADS and name not in FP8_WORKLOADS:
        print(f"unknown workload {name}; choose from {sorted(WORKLOADS) + sorted(FP8_WORKLOADS)}", file=sys.stderr)
        sys.exit(2)
    w = WORKLOADS.get(name) or FP8_WORKLOADS[name]
    if args.backward and w.dtype == "fp8":
        print("the backward pass takes fp16 or bf16 inputs", file=sys.stderr)
        sys.exit(2)
    if args.backward:
        backward_main(args, w)
        return
    ms, wall_ms = run_workload(w, args.steps, args.warmup, args.variant)
    stats = run_workload.last_stats
    tflops = w.flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = measured_traffic(w, args.variant)

    if args.all:
        print(f"{'workload':36s} {'ms':>9s} {'TFLOPS':>9s} {'%peak':>7s}", file=sys.stderr)
        for other in list(WORKLOADS.values()) + list(FP8_WORKLOADS.values()):
            oms, _ = run_workload(other, max(5, args.steps // 2), max(2, args.warmup // 2), args.variant)
            t = other.flops / (oms * 1e-3) / 1e12
            print(f"{other.name:36s} {oms:9.4f} {t:9.1f} {100 * t / PEAK_TFLOPS[other.dtype]:6.1f}%",
                  file=sys.stderr, flush=True)

    fp8 = w.dtype == "fp8"
    line = {
        "metric": FP8_METRIC if fp8 else METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else w.dtype,
        "data": ("synthetic (seeded N(0,1) inputs as E4M3 codes with one descale per tensor, bf16 output)" if fp8
                 else "synthetic (seeded N(0,1) inputs, rounded to the dtype)"),
        "config": {**w.describe(), "variant": args.variant, "parallelism": "single GPU",
                   "wall_ms_per_step": round(wall_ms, 5), "per_call": stats},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": traffic,
        },
    }
    probe = mfma_probe(fp8=fp8)
    if probe is not None:
        line["roofline"]["probe_peak"] = probe
        line["roofline"]["frac_probe"] = round(tflops / probe["value"], 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
