#!/usr/bin/env python3
"""Benchmark of the FP32 GEMM hot path (C = A.B, row-major) on one MI355X.

One step is one call of sgemm_mi355 on resident device inputs of the named
workload (default: square M = N = K = 8192, U[-1,1) from seed 4). Prints ONE
JSON line with GFLOP/s (2*M*N*K per call, GPU Parallel Book ch. 9, section
9.1), the fraction of the FP32 matrix peak, the roofline of the kernel, and
the CPU oracle timed on this host as a reported baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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
    if "_lds" in config_name:
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


def time_gpu(w, steps: int, warmup: int, kind: str, config, warmup_ms: float = 0.0):
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
        cid = sg.sgemm_mi355_select_config(w.M, w.N, w.K)
    else:
        cid = sg.sgemm_mi355_select_config_valu(w.M, w.N, w.K)

    def step():
        sg.matmul(Av, Bv, out=Cv, kind=kind, config=cid, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Optional extra warm-up by time: the engine clock ramps up over the first
    # tens of milliseconds of load after an idle gap.
    t_warm = time.perf_counter()
    while (time.perf_counter() - t_warm) * 1e3 < warmup_ms:
        step()
        torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = [s.elapsed_time(e) for s, e in zip(starts, ends)]  # ms
    total_ms = starts[0].elapsed_time(ends[-1])
    name = sg.sgemm_mi355_config_name(cid)
    return {
        "ms_per_step": total_ms / steps,
        "mean_launch_ms": sum(per_launch) / steps,
        "min_launch_ms": min(per_launch),
        "max_launch_ms": max(per_launch),
        "wall_s": wall,
        "config_name": name,
    }


def cpu_baseline(w, seconds: float):
    """The oracle (plain FP32 triple loop, OpenMP over rows), untuned, timed on
    this host on whole rows of the same workload until about `seconds` of work."""
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
    return {
        "value": round(gflops, 3),
        "unit": "GFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows_done} of {w.M} rows of C ({w.name}), {elapsed:.1f} s, "
                  f"{threads} OpenMP threads, affinity {len(os.sched_getaffinity(0))} cpus",
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
    ap.add_argument("--also", default="square4096",
                    help="comma-separated extra workloads reported under 'also' ('' for none)")
    ap.add_argument("--kind", default="mfma", choices=["mfma", "valu"])
    ap.add_argument("--config", default=None, help="force a kernel configuration by name")
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
    r = time_gpu(w, args.steps, args.warmup, args.kind, config)
    value = w.flops / (r["ms_per_step"] * 1e-3) / 1e9          # GFLOP/s, whole job (1 GPU)
    achieved = w.flops / (r["mean_launch_ms"] * 1e-3) / 1e12   # TFLOP/s per launch
    log(f"[bench] {r['config_name']}: {r['ms_per_step']:.3f} ms/step, {value:.1f} GFLOP/s")

    also = []
    for name in [s for s in args.also.split(",") if s and s != w.name]:
        wa = workloads.BY_NAME[name]
        ra = time_gpu(wa, max(args.steps, 20), args.warmup, args.kind, None, warmup_ms=300.0)
        va = wa.flops / (ra["ms_per_step"] * 1e-3) / 1e9
        also.append({"workload": wa.name, "value": round(va, 1), "unit": "GFLOP/s",
                     "ms_per_step": round(ra["ms_per_step"], 4), "config": ra["config_name"],
                     "frac_fp32_mfma_peak": round(va / (PEAK_MFMA_TFLOPS * 1e3), 4)})
        log(f"[bench] also {wa.name}: {va:.1f} GFLOP/s ({ra['config_name']})")

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
            "peak": PEAK_MFMA_TFLOPS if args.kind == "mfma" else PEAK_VECTOR_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
            "traffic": traffic,
            "kernel": r["config_name"],
            "mean_launch_ms": round(r["mean_launch_ms"], 4),
            "min_launch_ms": round(r["min_launch_ms"], 4),
            "max_launch_ms": round(r["max_launch_ms"], 4),
            "algorithmic_flops_per_launch": w.flops,
            "min_bytes_per_launch": w.min_bytes,
        },
        "also": also,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
