#!/usr/bin/env python3
"""Benchmark of the FP32 GEMM hot path (C = A.B, row-major) on one MI355X.

One step is one call of sgemm_mi355 on resident device inputs of the named
workload (default: square M = N = K = 8192, U[-1,1) from seed 4); the call
selects its kernel configuration from the actual pointers and leading
dimensions, as any caller's would. Prints ONE JSON line with GFLOP/s
(2*M*N*K per call, GPU Parallel Book ch. 9, section 9.1), the fraction of the
FP32 matrix peak, the roofline of the kernel, the same figures for the other
workloads under "also", and the CPU oracle timed on this host as a reported
baseline.

Timing: the timed calls are queued behind a spin kernel, so they run back to
back on the GPU and the host's cost per call (a ctypes call and the HIP
enqueue) stays out of the measurement; ms_per_step is the span of all steps
divided by their number, and the per-launch figures come from events around
each call, queued the same way.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks (dense): FP32 matrix 157.3 TFLOP/s (256 CU x 2.4 GHz
# x 256 FLOP/clk/CU); FP32 vector 157.3 TFLOP/s, which plain VOP2 v_fmac_f32
# with VGPR operands reaches on gfx950 (a throughput probe measured 143
# TFLOP/s; VOP3 v_fma_f32 with two scalar operands runs at half that rate);
# HBM3E 8 TB/s.
PEAK_MFMA_TFLOPS = 157.3
PEAK_VECTOR_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources(config_name: str):
    """The source files that define a configuration's kernel."""
    if config_name.startswith("valu"):
        return ("kernels_valu.hip", "sgemm_internal.h")
    if "_lds" in config_name or re.search(r"_rs\d*_sched", config_name):
        return ("kernels_mfma_dma.hip", "sgemm_internal.h")
    return ("kernels_mfma.hip", "sgemm_internal.h")


def kernel_source_hash(config_name: str) -> str:
    """Hash of the source files that define the configuration's kernel: counter
    figures taken on other sources no longer describe the kernel."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_fp32_matrix_02_amd", "csrc")
    for name in kernel_sources(config_name):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, config_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    e = table.get(f"{workload}/{config_name}")
    if not e or e.get("kernel_source_hash") != kernel_source_hash(config_name):
        return None
    return e.get("hbm_bytes_per_launch")


_SLEEP_CYCLES_PER_US = None


def queue_ahead(stream, us: float):
    """Enqueue a spin kernel of about `us` microseconds on `stream`, so the
    launches recorded after it are queued on the GPU before it ends: they then
    run back to back, and the host's per-launch cost (a ctypes call and the
    HIP enqueue, tens of microseconds) stays out of the timed region."""
    import torch

    global _SLEEP_CYCLES_PER_US
    if _SLEEP_CYCLES_PER_US is None:
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        s.record()
        torch.cuda._sleep(1_000_000)
        e.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_US = 1_000_000 / max(s.elapsed_time(e) * 1e3, 1.0)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(_SLEEP_CYCLES_PER_US * us))


def time_gpu(w, steps: int, warmup: int, kind: str, config, warmup_ms: float = 300.0):
    """Time `steps` calls of the path on resident inputs of workload w.

    Two timed passes, each behind queue_ahead: one pair of events around all
    steps (ms_per_step: the span of back-to-back launches divided by their
    number, the average launch duration including the gap between launches;
    a rocprofv3 kernel trace of the same run gives the kernel's own duration
    within that gap), then events around each call (the mean, least and
    largest single launch, each with its events' own overhead, a few
    microseconds that matter only for the smallest workloads). Without a
    forced configuration the call is sgemm_mi355 itself (sgemm_mi355_valu for
    the vector kind), which selects with the actual pointers and leading
    dimensions."""
    import torch
    import dense_fp32_matrix_02_amd as sg
    import workloads

    A, B = workloads.inputs(w)
    Ad = workloads.embed(A, w.lda).to("cuda") if w.lda != w.K else A.to("cuda")
    Bd = workloads.embed(B, w.ldb).to("cuda") if w.ldb != w.N else B.to("cuda")
    Cd = torch.empty((w.M, w.ldc), dtype=torch.float32, device="cuda")
    Av, Bv, Cv = Ad[:, :w.K], Bd[:, :w.N], Cd[:, :w.N]
    stream = torch.cuda.current_stream()
    if config is not None:
        cid = config
    elif kind == "mfma":
        cid = sg.sgemm_mi355_selected_config(w.M, w.N, w.K, Av.data_ptr(), w.lda, Bv.data_ptr(), w.ldb)
    else:
        cid = sg.sgemm_mi355_select_config_valu(w.M, w.N, w.K)

    def step():
        sg.matmul(Av, Bv, out=Cv, kind=kind, config=config, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Warm-up by time as well: after an idle gap (input generation on the
    # host) the engine clock takes tens of milliseconds of load to ramp up.
    t_warm = time.perf_counter()
    while (time.perf_counter() - t_warm) * 1e3 < warmup_ms:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    ahead_us = max(2000.0, 80.0 * steps)
    # pass 1: back-to-back throughput
    s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    queue_ahead(stream, ahead_us)
    s0.record(stream)
    for _ in range(steps):
        step()
    e0.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = s0.elapsed_time(e0)
    # pass 2: single launches
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    queue_ahead(stream, ahead_us)
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch = [s.elapsed_time(e) for s, e in zip(starts, ends)]  # ms
    return {
        "ms_per_step": total_ms / steps,
        "mean_launch_ms": sum(per_launch) / steps,
        "min_launch_ms": min(per_launch),
        "max_launch_ms": max(per_launch),
        "wall_s": wall,
        "config_name": sg.sgemm_mi355_config_name(cid),
    }


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_gflops(w, threads: int, reps: int) -> float:
    """The oracle on the whole of workload w (median of `reps` runs) with
    `threads` OpenMP threads, in GFLOP/s."""
    import numpy as np
    import oracle
    import workloads

    A, B = workloads.inputs(w)
    A, B = workloads.as_numpy(A), workloads.as_numpy(B)
    out = np.empty((w.M, w.N), np.float32)
    n0 = oracle.max_threads()
    oracle.set_threads(threads)
    try:
        times = []
        for _ in range(reps):
            t = time.perf_counter()
            oracle.sgemm_f32(A, B, out=out)
            times.append(time.perf_counter() - t)
    finally:
        oracle.set_threads(n0)
    times.sort()
    return w.flops / times[len(times) // 2] / 1e9


def cpu_baseline(w, seconds: float, others=()):
    """The oracle (plain FP32 triple loop, OpenMP over rows), untuned, timed on
    this host: on whole rows of workload w until about `seconds` of work (the
    reported value), then on every workload in `others` whole (median of 3
    runs for those under 1e10 FLOP), and single-threaded on those under 3e9
    FLOP."""
    import numpy as np
    import oracle
    import workloads

    A, B = workloads.inputs(w)
    A, B = workloads.as_numpy(A), workloads.as_numpy(B)
    threads = oracle.max_threads()
    rows_done, elapsed, chunk = 0, 0.0, 16
    while rows_done < w.M and elapsed < seconds:
        r = min(chunk, w.M - rows_done)
        a = np.ascontiguousarray(A[rows_done:rows_done + r])
        t = time.perf_counter()
        oracle.sgemm_f32(a, B)
        elapsed += time.perf_counter() - t
        rows_done += r
        chunk = min(chunk * 2, 512)
    gflops = 2.0 * rows_done * w.N * w.K / elapsed / 1e9
    per_workload = []
    for wo in others:
        reps = 3 if wo.flops < 1e10 else 1
        entry = {"workload": wo.name, "GFLOP/s": round(oracle_gflops(wo, threads, reps), 3),
                 "threads": threads, "runs": reps}
        if wo.flops < 3e9:
            entry["GFLOP/s_1_thread"] = round(oracle_gflops(wo, 1, 3), 3)
        per_workload.append(entry)
    return {
        "value": round(gflops, 3),
        "unit": "GFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows_done} of {w.M} rows of C ({w.name}), {elapsed:.1f} s, "
                  f"{threads} OpenMP threads, affinity {len(os.sched_getaffinity(0))} cpus",
        "cpu_model": cpu_model(),
        "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "per_workload": per_workload,
    }


def copy_probe(nbytes: int, steps: int):
    """Plain device copy of a known number of bytes (read nbytes, write nbytes)
    per launch, timed with events; the HBM counters of this kernel give the
    scale factor from counter units to bytes."""
    import torch

    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        torch.mul(src, 1.0, out=dst)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                      "ms_per_copy": round(ms, 4), "GBps_read_plus_write": round(8 * n / ms / 1e6, 1)}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="square8192")
    ap.add_argument("--also", default="square256,square1024,square4096,ragged3001x2047x1537",
                    help="comma-separated extra workloads reported under 'also' ('' for none)")
    ap.add_argument("--kind", default="mfma", choices=["mfma", "valu"])
    ap.add_argument("--config", default=None, help="force a kernel configuration by name")
    ap.add_argument("--warmup-ms", type=float, default=300.0,
                    help="extra warm-up by time before each workload's timed steps (engine clock ramp)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="instead of the GEMM, run `steps` plain device copies of BYTES bytes "
                         "(reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this GEMM has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_fp32_matrix_02_amd as sg
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    sg.load()
    w = workloads.BY_NAME[args.workload]
    config = sg.config_id(args.config) if args.config else None

    log(f"[bench] {w.name} M={w.M} N={w.N} K={w.K} kind={args.kind} steps={args.steps} warmup={args.warmup}")
    peak = PEAK_MFMA_TFLOPS if args.kind == "mfma" else PEAK_VECTOR_TFLOPS
    r = time_gpu(w, args.steps, args.warmup, args.kind, config, args.warmup_ms)
    value = w.flops / (r["ms_per_step"] * 1e-3) / 1e9          # GFLOP/s, whole job (1 GPU)
    achieved = w.flops / (r["ms_per_step"] * 1e-3) / 1e12      # TFLOP/s per launch (back-to-back span)
    log(f"[bench] {r['config_name']}: {r['ms_per_step']:.4f} ms/step, {value:.1f} GFLOP/s, "
        f"mean launch {r['mean_launch_ms']:.4f} ms")

    also = []
    others = [workloads.BY_NAME[n] for n in args.also.split(",") if n and n != w.name]
    for wa in others:
        ra = time_gpu(wa, max(args.steps, 20), args.warmup, args.kind, None, args.warmup_ms)
        va = wa.flops / (ra["ms_per_step"] * 1e-3) / 1e9
        ka = wa.flops / (ra["ms_per_step"] * 1e-3) / 1e12
        also.append({"workload": wa.name, "M": wa.M, "N": wa.N, "K": wa.K, "value": round(va, 1),
                     "unit": "GFLOP/s", "ms_per_step": round(ra["ms_per_step"], 5), "kernel": ra["config_name"],
                     "event_launch_ms": round(ra["mean_launch_ms"], 5),
                     "event_launch_min_ms": round(ra["min_launch_ms"], 5),
                     "frac_fp32_mfma_peak": round(va / (PEAK_MFMA_TFLOPS * 1e3), 4),
                     "frac_fp32_vector_peak": round(va / (PEAK_VECTOR_TFLOPS * 1e3), 4),
                     "launch_tflops": round(ka, 2), "launch_frac": round(ka / peak, 4),
                     "traffic": stored_traffic(wa.name, ra["config_name"])})
        log(f"[bench] also {wa.name}: {va:.1f} GFLOP/s, {ra['ms_per_step'] * 1e3:.2f} us per launch "
            f"({ra['config_name']})")

    traffic = stored_traffic(w.name, r["config_name"])
    out = {
        "metric": "SGEMM GFLOP/s (FP32) at N=4096/8192; % of MI355X FP32 peak",
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "lda": w.lda, "ldb": w.ldb,
                   "ldc": w.ldc, "dist": w.dist, "seed": w.seed, "kernel": r["config_name"],
                   "kind": args.kind},
        "frac_fp32_mfma_peak": round(value / (PEAK_MFMA_TFLOPS * 1e3), 4),
        "frac_fp32_vector_peak": round(value / (PEAK_VECTOR_TFLOPS * 1e3), 4),
        "peaks_tflops": {"fp32_mfma": PEAK_MFMA_TFLOPS, "fp32_vector": PEAK_VECTOR_TFLOPS},
        "roofline": {
            "bound": "mfma" if args.kind == "mfma" else "alu",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel": r["config_name"],
            "launch_ms": round(r["ms_per_step"], 4),
            "event_launch_ms": round(r["mean_launch_ms"], 4),
            "event_launch_min_ms": round(r["min_launch_ms"], 4),
            "event_launch_max_ms": round(r["max_launch_ms"], 4),
            "algorithmic_flops_per_launch": w.flops,
            "min_bytes_per_launch": w.min_bytes,
        },
        "also": also,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle for about {args.cpu_seconds:.0f} s, then on the other workloads")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, others)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
