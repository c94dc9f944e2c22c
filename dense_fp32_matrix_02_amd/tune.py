"""Tile-configuration tuner: time every kernel configuration on each problem
shape and emit the tile table the library compiles in.

The best tile is found by measurement, not derived (CUDA Handbook section
17.3 sweeps the microtile; GPU Parallel Book ch. 9, section 9.6 sweeps the
occupancy setting). For each shape every matrix-core configuration runs on
seeded U[-1,1) inputs; the median of `reps` event-timed launches decides.

    python -m dense_fp32_matrix_02_amd.tune [--shapes 8192x8192x8192,...]
        [--reps 20] [--json results.json] [--table tile_table.inc]

``--table`` writes a tile_table.inc with one exact-shape entry per measured
shape; copy it to csrc/ and rebuild to use it.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TABLE_HEADER = """\
// Tile-configuration table: which kernel configuration each problem shape
// uses. The best tile is an empirical question (CUDA Handbook section 17.3:
// the microtile is chosen by sweeping; GPU Parallel Book section 9.6: the
// occupancy setting is found by measurement), so each entry records the
// fastest configuration measured on MI355X for one shape. A shape without
// its own entry takes the nearest measured shape (in log M, log N, log K,
// within a factor of two in each), else the rule in sgemm_api.hip.
//
// Written by dense_fp32_matrix_02_amd/tune.py (median of {reps} launches per
// configuration). Format: {{M, N, K, "configuration name"}}.
static const ShapeEntry kShapeTable[] = {{
"""


def parse_shapes(text):
    out = []
    for s in text.split(","):
        s = s.strip()
        if s:
            M, N, K = (int(x) for x in s.lower().split("x"))
            out.append((M, N, K))
    return out


def time_config(M, N, K, cid, reps, warmup, A, B, C):
    import torch
    import dense_fp32_matrix_02_amd as sg

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        sg.matmul(A, B, out=C, config=cid, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for s, e in ev:
        s.record(stream)
        sg.matmul(A, B, out=C, config=cid, stream=stream)
        e.record(stream)
    torch.cuda.synchronize()
    return statistics.median(s.elapsed_time(e) for s, e in ev)


def main(argv=None):
    import torch
    import dense_fp32_matrix_02_amd as sg
    import workloads

    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--shapes", default=",".join(f"{w.M}x{w.N}x{w.K}" for w in workloads.WORKLOADS))
    ap.add_argument("--grid", action="store_true",
                    help="also measure the grid M, N in {128..8192} (powers of two) x K in {256, 1024, 4096, 16384}")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--kinds", default="mfma", help="mfma, valu or mfma,valu")
    ap.add_argument("--splitk", default="", help="split counts to time with sgemm_mi355_splitk, e.g. 2,4,8")
    ap.add_argument("--json", default=None)
    ap.add_argument("--table", default=None)
    args = ap.parse_args(argv)

    names = sg.config_names()
    kinds = args.kinds.split(",")
    cands = [i for i, n in enumerate(names)
             if n.startswith(tuple(kinds)) and sg.sgemm_mi355_config_ops(i) == (0, 0)]
    results = []
    shapes = parse_shapes(args.shapes)
    if args.grid:
        # Every M, N in [64, 16384] and K in [128, 32768] lies within a factor
        # of two of a grid point in each dimension (the table's lookup radius).
        sides = [128, 256, 512, 1024, 2048, 4096, 8192]
        shapes += [(m, n, k) for m in sides for n in sides for k in (256, 1024, 4096, 16384)
                   if (m, n, k) not in shapes]
    for (M, N, K) in shapes:
        A, B = workloads.draw(M, N, K, 1234, "uniform")
        Ad, Bd = A.to("cuda"), B.to("cuda")
        C = torch.empty((M, N), device="cuda")
        row = {"M": M, "N": N, "K": K, "times_ms": {}}
        for cid in cands:
            ms = time_config(M, N, K, cid, args.reps, args.warmup, Ad, Bd, C)
            row["times_ms"][names[cid]] = ms
            print(f"{M}x{N}x{K} {names[cid]:28s} {ms:9.4f} ms {2 * M * N * K / ms / 1e9:9.2f} TFLOP/s",
                  flush=True)
        for sp in [int(x) for x in args.splitk.split(",") if x]:
            need = sg.sgemm_mi355_splitk_workspace_size(M, N, K, sp)
            ws = torch.empty((need + 3) // 4 + 1, device="cuda")
            stream = torch.cuda.current_stream()
            run = lambda: sg.gemm_splitk(Ad, Bd, C, splits=sp, workspace=ws, stream=stream)
            for _ in range(args.warmup):
                run()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.reps)]
            for s0, e0 in ev:
                s0.record(stream)
                run()
                e0.record(stream)
            torch.cuda.synchronize()
            ms = statistics.median(s0.elapsed_time(e0) for s0, e0 in ev)
            row.setdefault("splitk_ms", {})[sp] = ms
            print(f"{M}x{N}x{K} splitk={sp:<3d} (gemm + reduce)        {ms:9.4f} ms "
                  f"{2 * M * N * K / ms / 1e9:9.2f} TFLOP/s", flush=True)
        mfma = {n: t for n, t in row["times_ms"].items() if n.startswith("mfma")}
        if mfma:
            row["best"] = min(mfma, key=mfma.get)
            row["default"] = names[sg.sgemm_mi355_select_config(M, N, K)]
            print(f"  best {row['best']}  (table/rule picks {row['default']})", flush=True)
        results.append(row)
        del Ad, Bd, C
    if args.json:
        with open(args.json, "w") as f:
            json.dump(results, f, indent=1)
    if args.table:
        with open(args.table, "w") as f:
            f.write(TABLE_HEADER.format(reps=args.reps))
            for r in results:
                if "best" in r:
                    f.write(f'    {{{r["M"]}, {r["N"]}, {r["K"]}, "{r["best"]}"}},\n')
            f.write("    {0, 0, 0, nullptr},  // sentinel\n};\n")


if __name__ == "__main__":
    main()
