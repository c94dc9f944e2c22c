"""Tile-configuration tuner: time every kernel configuration on each problem
shape and emit the tile table the library compiles in.

The best tile is found by measurement, not derived (CUDA Handbook section
17.3 sweeps the microtile; GPU Parallel Book ch. 9, section 9.6 sweeps the
occupancy setting). For each shape every matrix-core configuration runs on
seeded U[-1,1) inputs; the median of `reps` event-timed launches decides.

    python -m dense_fp32_matrix_02_amd.tune [--shapes 8192x8192x8192,...]
        [--reps 20] [--json results.json] [--table tile_table.inc]
        [--ops nn|tn|nt|tt] [--batch B]

``--table`` writes a tile_table.inc with one exact-shape entry per measured
shape; copy it to csrc/ and rebuild to use it. ``--ops`` times the
configurations built for transposed operands (op(A) = A^T for a first letter
t, op(B) = B^T for a second), on operands stored transposed; ``--batch``
times strided batches of B independent products per launch. The table holds
plain single products only, so ``--table`` needs the defaults of both.
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
// fastest register-staged configuration measured on MI355X for one shape
// (the direct-to-LDS kernel is chosen by rule on top, for problems that
// qualify). A shape without its own entry takes the nearest measured shape
// (in log M, log N, log K, within a factor of two in each), else the rule in
// sgemm_api.hip.
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


def time_call(call, reps, warmup):
    """Median of `reps` event-timed calls after `warmup` untimed ones (ms)."""
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        call(stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for s, e in ev:
        s.record(stream)
        call(stream)
        e.record(stream)
    torch.cuda.synchronize()
    return statistics.median(s.elapsed_time(e) for s, e in ev)


def make_inputs(M, N, K, opA, opB, batch):
    """Device operands for one shape: op(A) is M x K and op(B) is K x N, stored
    transposed for a T op; with batch > 1, `batch` independent entries."""
    import torch
    import workloads

    def one(seed):
        A, B = workloads.draw(M, N, K, seed, "uniform")
        A = A.t().contiguous() if opA else A
        B = B.t().contiguous() if opB else B
        return A, B

    if batch == 1:
        A, B = one(1234)
        return A.to("cuda"), B.to("cuda"), torch.empty((M, N), device="cuda")
    pairs = [one(1234 + b) for b in range(batch)]
    A = torch.stack([p[0] for p in pairs]).to("cuda")
    B = torch.stack([p[1] for p in pairs]).to("cuda")
    return A, B, torch.empty((batch, M, N), device="cuda")


def config_call(A, B, C, cid, opA, opB, batch):
    import dense_fp32_matrix_02_amd as sg

    if batch == 1 and not opA and not opB:
        return lambda stream: sg.matmul(A, B, out=C, config=cid, stream=stream)
    if batch == 1:
        return lambda stream: sg.gemm(A, B, C, opA=opA, opB=opB, config=cid, stream=stream)
    return lambda stream: sg.gemm_strided_batched(A, B, C, opA=opA, opB=opB, config=cid, stream=stream)


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
    ap.add_argument("--from-json", default=None, metavar="JSON",
                    help="write --table from a saved --json result instead of measuring")
    ap.add_argument("--ops", default="nn", choices=["nn", "tn", "nt", "tt"])
    ap.add_argument("--batch", type=int, default=1)
    args = ap.parse_args(argv)
    opA, opB = int(args.ops[0] == "t"), int(args.ops[1] == "t")
    if args.table and (opA or opB or args.batch != 1):
        ap.error("--table records plain single products: leave --ops and --batch at their defaults")
    if args.splitk and (opA or opB or args.batch != 1):
        ap.error("--splitk times plain single products")

    if args.from_json:
        with open(args.from_json) as f:
            write_table(json.load(f), args.table, args.reps)
        return

    names = sg.config_names()
    kinds = args.kinds.split(",")
    cands = [i for i, n in enumerate(names)
             if n.startswith(tuple(kinds)) and sg.sgemm_mi355_config_ops(i) == (opA, opB)]
    results = []
    shapes = parse_shapes(args.shapes)
    if args.grid:
        # Every M, N in [64, 16384] and K in [128, 32768] lies within a factor
        # of two of a grid point in each dimension (the table's lookup radius).
        sides = [128, 256, 512, 1024, 2048, 4096, 8192]
        shapes += [(m, n, k) for m in sides for n in sides for k in (256, 1024, 4096, 16384)
                   if (m, n, k) not in shapes]
    tag = ("" if args.ops == "nn" else f" {args.ops}") + ("" if args.batch == 1 else f" x{args.batch}")
    for (M, N, K) in shapes:
        Ad, Bd, C = make_inputs(M, N, K, opA, opB, args.batch)
        row = {"M": M, "N": N, "K": K, "ops": args.ops, "batch": args.batch, "times_ms": {}}
        flops = 2 * M * N * K * args.batch
        for cid in cands:
            ms = time_call(config_call(Ad, Bd, C, cid, opA, opB, args.batch), args.reps, args.warmup)
            row["times_ms"][names[cid]] = ms
            print(f"{M}x{N}x{K}{tag} {names[cid]:28s} {ms:9.4f} ms {flops / ms / 1e9:9.2f} TFLOP/s",
                  flush=True)
        for sp in [int(x) for x in args.splitk.split(",") if x]:
            need = sg.sgemm_mi355_splitk_workspace_size(M, N, K, sp)
            ws = torch.empty((need + 3) // 4 + 1, device="cuda")
            ms = time_call(lambda stream: sg.gemm_splitk(Ad, Bd, C, splits=sp, workspace=ws, stream=stream),
                           args.reps, args.warmup)
            row.setdefault("splitk_ms", {})[sp] = ms
            print(f"{M}x{N}x{K} splitk={sp:<3d} (gemm + reduce)        {ms:9.4f} ms "
                  f"{2 * M * N * K / ms / 1e9:9.2f} TFLOP/s", flush=True)
        mfma = {n: t for n, t in row["times_ms"].items() if n.startswith("mfma")}
        if mfma:
            row["best"] = min(mfma, key=mfma.get)
            row["default"] = names[sg.sgemm_mi355_select_config_ex(opA, opB, M, N, K, args.batch)]
            print(f"  best {row['best']}  (table/rule picks {row['default']})", flush=True)
        results.append(row)
        del Ad, Bd, C
    if args.json:
        with open(args.json, "w") as f:
            json.dump(results, f, indent=1)
    if args.table:
        write_table(results, args.table, args.reps)


def write_table(results, path, reps):
    """One entry per measured shape: the fastest register-staged configuration.
    Direct-to-LDS configurations (_lds) are left out: the library switches to
    them by rule, only for problems that qualify for direct loads, so a
    nearest-shape lookup never lands on one for a problem that does not."""
    with open(path, "w") as f:
        f.write(TABLE_HEADER.format(reps=reps))
        for r in results:
            t = {n: ms for n, ms in r["times_ms"].items() if n.startswith("mfma") and "_lds" not in n}
            if t:
                f.write(f'    {{{r["M"]}, {r["N"]}, {r["K"]}, "{min(t, key=t.get)}"}},\n')
        f.write("    {0, 0, 0, nullptr},  // sentinel\n};\n")


if __name__ == "__main__":
    main()
