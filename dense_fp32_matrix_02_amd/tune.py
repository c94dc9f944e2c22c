"""Tile-configuration tuner: time every kernel configuration on each problem
shape and emit the tile table the library compiles in.

The best tile is found by measurement, not derived (CUDA Handbook section
17.3 sweeps the microtile; GPU Parallel Book ch. 9, section 9.6 sweeps the
occupancy setting). For each shape every matrix-core configuration built for
the op pair runs on seeded U[-1,1) inputs; the time per launch of `reps`
launches run back to back (as bench.py times them) is recorded, with each
configuration's occupancy (workgroups per compute unit, from the HIP
runtime).

    python -m dense_fp32_matrix_02_amd.tune [--shapes 8192x8192x8192,...]
        [--grid | --smallk-grid] [--reps 20] [--json results.json] [--table tile_table.inc]
        [--ops nn|tn|nt|tt] [--batch B]
    python -m dense_fp32_matrix_02_amd.tune --from-json nn.json,tn.json,nt.json,tt.json \
        --table dense_fp32_matrix_02_amd/csrc/tile_table.inc

``--ops`` times the configurations built for transposed operands (op(A) =
A^T for a first letter t, op(B) = B^T for a second), on operands stored
transposed; ``--batch`` times strided batches of B independent products per
launch. ``--table`` writes the table from the single products measured (this
run's, or the saved ``--from-json`` results of one file per op pair); copy it
to csrc/ and rebuild to use it.
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
// Tile-configuration table: measured run times of the kernel configurations
// on a grid of problem shapes, per op pair. The best tile is an empirical
// question (CUDA Handbook section 17.3: the microtile is chosen by sweeping;
// GPU Parallel Book section 9.6: the occupancy setting is found by
// measurement). The selection takes the measured shape nearest a problem (in
// log M, log N, log K, within a factor of two in each) and scales each
// configuration's time there to the problem with a model of how its
// workgroups fill the compute units (sgemm_api.hip); the fastest predicted
// configuration runs.
//
// Per op pair: the candidates (configurations that are the fastest on at
// least one measured shape, overall or among those without direct loads, so
// that misaligned problems have register-staged candidates) with their
// occupancy (workgroups one compute unit holds, from the HIP runtime), then
// per shape {{M, N, K}} and the
// candidates' times per launch in microseconds; 0 marks a time more than
// {cut}x the shape's best (never a candidate there). Then every
// configuration of the op pair with its occupancy and its median time per
// unit of modelled busy time over the shapes: the selection's estimate for
// batches and for problems with no measured shape nearby. Where stream-K forms
// were timed (a grid of shapes whose tiles leave a partial last round), each
// one's time per slab of the evenly dealt work beyond a fixed overhead,
// median over those shapes (sgemm_mi355_select_streamk). A last block records,
// per shape of a second grid, the fastest split count of sgemm_mi355_splitk,
// which sgemm_mi355_select_splitk suggests for shapes near it.
//
// Written by dense_fp32_matrix_02_amd/tune.py (time per launch of {reps}
// launches run back to back, per configuration and shape{passes}).
"""

# Times more than this factor above a shape's best are stored as 0 (not a
# candidate at that shape): the fill model never scales one configuration
# against another by as much at a neighbouring shape.
TABLE_CUT = 2.0
OPS_NAMES = ("nn", "nt", "tn", "tt")
# The split-K grid: shapes whose tile grids leave compute units idle, and K
# long enough for splitting to be worth a second pass.
SPLIT_SIDES = (64, 96, 128, 192, 256, 384, 512, 768, 1024, 1536, 2048, 3072)
# The stream-K grid: single products whose tile counts leave a partial last
# round for every stream-K tile (M, N multiples of 4 and K of 16, so every op
# pair takes the direct path), from long K on small M x N to large cubes.
STREAMK_SHAPES = ((5120, 5120, 5120), (6144, 6144, 6144), (3072, 3072, 8192), (10240, 10240, 2048),
                  (4608, 4608, 4608), (2560, 2560, 8192), (3328, 3328, 8192), (7168, 7168, 4096),
                  (2048, 2048, 8192), (2048, 2048, 4096), (1536, 1536, 16384), (1024, 1024, 16384),
                  (2048, 2048, 2048), (768, 768, 65536), (3584, 3584, 3584), (2816, 2816, 5632),
                  (4352, 4352, 2048), (1280, 1280, 32768), (5120, 2560, 6144))
# Fixed cost of a stream-K call beyond its slabs (kStreamKOverheadUs in
# sgemm_api.hip): the partial sums (two BM x BN blocks per workgroup, 128 MiB
# for every stream-K tile on 256 compute units), the fixup kernel and its launch.
STREAMK_OVERHEAD_US = 40.0
# The selection considers stream-K only for K from half the grid's smallest K
# (kStreamKMinK in sgemm_api.hip): the time per slab is not carried further.
STREAMK_MIN_K = min(k for _, _, k in STREAMK_SHAPES) // 2
SPLIT_KS = (1024, 2048, 4096, 8192, 16384, 32768, 65536)
# The side lengths of the plain grid and of the short-K grid, and the plain
# grid's depths.
GRID_SIDES = (128, 256, 512, 1024, 2048, 4096, 8192)
GRID_KS = (256, 1024, 4096, 16384)
# The short-K grid: products whose K is a few slabs, where the launch and the
# store of C take much of the time. Their launches last microseconds, so they
# are timed with more repetitions than the default, in two passes (a slow
# spell of a tenth of a millisecond once doubled one configuration's time in
# one row, 14 us against 7 at its neighbours).
SMALLK_KS = (32, 96)
SMALLK_REPS = 30
SMALLK_WARMUP = 10
SMALLK_PASSES = 2


def time_passes(names, passes, timer):
    """{name: least of `passes` timings}: each pass times every name in order
    with timer(name), so a slow spell hits one configuration's passes only if
    it lasts through the others' timings in between."""
    best = {}
    for _ in range(passes):
        for name in names:
            ms = timer(name)
            best[name] = min(ms, best.get(name, ms))
    return best


def parse_shapes(text):
    out = []
    for s in text.split(","):
        s = s.strip()
        if s:
            M, N, K = (int(x) for x in s.lower().split("x"))
            out.append((M, N, K))
    return out


_SLEEP_CYCLES_PER_US = None
# Host time to issue one call, covered by the spin kernel queued ahead of the
# timed calls (a ctypes call and a HIP enqueue take tens of microseconds).
_ISSUE_US = 80.0


def _queue_ahead(stream, us):
    """Enqueue a spin kernel of about `us` microseconds on `stream`, so the
    calls issued after it wait on the GPU and then run back to back."""
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


def time_call(call, reps, warmup):
    """Time per call (ms) of `reps` calls run back to back between one pair of
    events, after `warmup` untimed ones: the calls are queued behind a spin
    kernel, so the host's issue cost stays out. This is how bench.py times a
    workload; an event pair around each call adds a few microseconds per
    call, more for some kernels than for others."""
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        call(stream)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _queue_ahead(stream, _ISSUE_US * reps)
    s.record(stream)
    for _ in range(reps):
        call(stream)
    e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


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
    ap.add_argument("--smallk-grid", action="store_true",
                    help="measure the grid M, N in {128..8192} (powers of two) x K in {32, 96}, with at least "
                         f"{SMALLK_REPS} repetitions, {SMALLK_WARMUP} warm-up launches and {SMALLK_PASSES} passes "
                         "(launches of a few microseconds)")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--passes", type=int, default=1,
                    help="time each shape's configurations this many times over, keeping each one's least time")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--kinds", default="mfma", help="mfma, valu or mfma,valu")
    ap.add_argument("--splitk", default="", help="split counts to time with sgemm_mi355_splitk, e.g. 2,4,8")
    ap.add_argument("--streamk", action="store_true",
                    help="also time the stream-K form of every configuration that has one")
    ap.add_argument("--selected", action="store_true",
                    help="time only the configuration the library selects for each shape")
    ap.add_argument("--streamk-grid", action="store_true",
                    help="time plain and stream-K forms on the stream-K grid (for --table)")
    ap.add_argument("--splitk-grid", action="store_true",
                    help="time split counts 1..64 on the grid M, N in {64..3072} (powers of two and 1.5x them) x K in {1024..65536} "
                         "(powers of two) for the table's split-K block (no per-configuration timings)")
    ap.add_argument("--json", default=None)
    ap.add_argument("--table", default=None)
    ap.add_argument("--from-json", default=None, metavar="JSON[,JSON...]",
                    help="write --table from saved --json results (one file per op pair, plus the "
                         "split-K grid) instead of measuring")
    ap.add_argument("--ops", default="nn", choices=["nn", "tn", "nt", "tt"])
    ap.add_argument("--batch", type=int, default=1)
    args = ap.parse_args(argv)
    opA, opB = int(args.ops[0] == "t"), int(args.ops[1] == "t")
    if args.passes < 1:
        ap.error("--passes must be at least 1")
    if args.from_json and not args.table:
        ap.error("--from-json writes a table: give --table")
    if args.table and args.batch != 1:
        ap.error("--table records single products: leave --batch at 1")
    if args.splitk and (opA or opB or args.batch != 1):
        ap.error("--splitk times plain single products")

    if args.splitk_grid:
        if opA or opB or args.batch != 1 or args.grid:
            ap.error("--splitk-grid times plain single products on its own grid")
        args.kinds = "none"
        args.splitk = "1,2,4,8,16,32,64"
        args.shapes = ",".join(f"{m}x{n}x{k}" for m in SPLIT_SIDES for n in SPLIT_SIDES for k in SPLIT_KS)
    if args.smallk_grid:
        if args.batch != 1 or args.grid:
            ap.error("--smallk-grid times single products on its own grid")
        args.reps = max(args.reps, SMALLK_REPS)
        args.warmup = max(args.warmup, SMALLK_WARMUP)
        args.passes = max(args.passes, SMALLK_PASSES)
        args.shapes = ",".join(f"{m}x{n}x{k}" for m in GRID_SIDES for n in GRID_SIDES for k in SMALLK_KS)
    if args.streamk_grid:
        if args.batch != 1 or args.grid:
            ap.error("--streamk-grid times single products on its own grid")
        args.streamk = True
        args.shapes = ",".join(f"{m}x{n}x{k}" for m, n, k in STREAMK_SHAPES)
    if args.from_json:
        results = []
        for path in args.from_json.split(","):
            with open(path) as f:
                results += json.load(f)
        write_table(results, args.table, args.reps)
        return

    names = sg.config_names()
    kinds = args.kinds.split(",")
    cands = [i for i, n in enumerate(names)
             if n.startswith(tuple(kinds)) and sg.sgemm_mi355_config_ops(i) == (opA, opB)]
    results = []
    shapes = parse_shapes(args.shapes)
    if args.grid:
        # Every M, N in [64, 16384] and K in [128, 32768] lies within a factor
        # of two of a grid point in each dimension (the table's lookup radius);
        # the short-K grid extends K down to 16.
        shapes += [(m, n, k) for m in GRID_SIDES for n in GRID_SIDES for k in GRID_KS
                   if (m, n, k) not in shapes]
    # stream-K forms are timed whatever --kinds says
    sk_cands = [i for i in range(len(names)) if sg.sgemm_mi355_config_streamk(i) == 1
                and sg.sgemm_mi355_config_ops(i) == (opA, opB)] if args.streamk else []
    occupancy = {names[cid]: sg.sgemm_mi355_config_occupancy(cid) for cid in cands + sk_cands}
    tag = ("" if args.ops == "nn" else f" {args.ops}") + ("" if args.batch == 1 else f" x{args.batch}")
    for (M, N, K) in shapes:
        Ad, Bd, C = make_inputs(M, N, K, opA, opB, args.batch)
        row = {"M": M, "N": N, "K": K, "ops": args.ops, "batch": args.batch, "reps": args.reps,
               "passes": args.passes, "times_ms": {},
               "occupancy": occupancy, "streamk_grid": bool(args.streamk_grid)}
        flops = 2 * M * N * K * args.batch
        shape_cands = [sg.sgemm_mi355_select_config_ex(opA, opB, M, N, K, args.batch)] if args.selected else cands
        row["times_ms"].update(time_passes(
            [names[cid] for cid in shape_cands], args.passes,
            lambda name: time_call(config_call(Ad, Bd, C, sg.config_id(name), opA, opB, args.batch),
                                   args.reps, args.warmup)))
        for cid in shape_cands:
            ms = row["times_ms"][names[cid]]
            print(f"{M}x{N}x{K}{tag} {names[cid]:28s} {ms:9.4f} ms {flops / ms / 1e9:9.2f} TFLOP/s",
                  flush=True)
        if args.streamk and args.batch == 1:
            for cid in sk_cands:
                need = sg.sgemm_mi355_streamk_workspace_size(opA, opB, M, N, K, cid)
                ws = torch.empty((need + 3) // 4 + 4, device="cuda")
                ms = time_call(lambda stream, cid=cid: sg.gemm_streamk(Ad, Bd, C, opA=opA, opB=opB, workspace=ws,
                                                                       config=cid, stream=stream),
                               args.reps, args.warmup)
                row.setdefault("streamk_ms", {})[names[cid]] = ms
                print(f"{M}x{N}x{K}{tag} streamk {names[cid]:28s} {ms:9.4f} ms {flops / ms / 1e9:9.2f} TFLOP/s",
                      flush=True)
                del ws
            sel = sg.sgemm_mi355_select_streamk(opA, opB, M, N, K)
            row["streamk_choice"] = names[sel] if sel >= 0 else None
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
            print(f"  best {row['best']}  (selection picks {row['default']})", flush=True)
        results.append(row)
        del Ad, Bd, C
    if args.json:
        with open(args.json, "w") as f:
            json.dump(results, f, indent=1)
    if args.table:
        write_table(results, args.table, args.reps)


# Fill model of the selection (busy_time in csrc/sgemm_api.hip): the busiest
# compute unit's share of workgroups, stretched while fewer than SAT_CHAINS
# 32x32 accumulator blocks are resident, times the slab count plus the store
# of C as STORE_DEPTH / BK more slabs (a CU's share of HBM bandwidth writes a
# tile in the time its share of the peak spends on about 40 steps of k).
SAT_CHAINS = 8
STORE_DEPTH = 40.0


def busy_time(bm, bn, bk, kgroups, occ, M, N, K, batch=1):
    wgs = -(-M // bm) * -(-N // bn) * min(batch, 65535)
    n = -(-wgs // 256)
    resident = min(n, occ) * kgroups * (bm // 32) * (bn // 32)
    stretch = 1.0 if resident >= SAT_CHAINS else SAT_CHAINS / resident
    return n * stretch * (-(-K // bk) + STORE_DEPTH / bk)


def config_geometry(name):
    """(bm, bn, bk, kgroups) of a configuration of the built library."""
    import re

    import dense_fp32_matrix_02_amd as sg

    bm, bn, bk, _ = sg.sgemm_mi355_config_info(sg.config_id(name))
    kg = re.search(r"_kg(\d+)", name)
    return bm, bn, bk, int(kg.group(1)) if kg else 1


def streamk_norms(rows, occ):
    """{name: (occupancy, microseconds per slab)} for the stream-K forms timed
    in `rows`: per configuration, the median over shapes where its direct
    kernel splits tiles of (time - STREAMK_OVERHEAD_US) / (tiles * (slabs +
    STORE_DEPTH / BK) / 256), slabs counting a partial last one and the store
    of each tile counted as in busy_time."""
    import dense_fp32_matrix_02_amd as sg

    known = set(sg.config_names())
    per = {}
    for r in rows:
        M, N, K = r["M"], r["N"], r["K"]
        for n, ms in r["streamk_ms"].items():
            if n not in known or n not in occ:
                continue
            cid = sg.config_id(n)
            bm, bn, bk, _ = sg.sgemm_mi355_config_info(cid)
            opA, opB = sg.sgemm_mi355_config_ops(cid)
            # the tuner's operands are contiguous, so a leading dimension is a row length
            direct = K >= bk and (M % 4 == 0 if opA else K % 4 == 0) and (K % 4 == 0 if opB else N % 4 == 0)
            if not direct:
                continue  # register-staged kernel
            tiles = -(-M // bm) * -(-N // bn)
            if tiles % (256 * occ[n]) == 0:
                continue  # whole rounds: the plain launch ran
            slabs = tiles * (-(-K // bk) + STORE_DEPTH / bk) / 256
            per.setdefault(n, []).append((ms * 1e3 - STREAMK_OVERHEAD_US) / slabs)
    return {n: (occ[n], statistics.median(v)) for n, v in sorted(per.items())}


def write_table(results, path, reps):
    """The tile table from single-product rows of any op pairs: per op pair,
    the configurations that are fastest on at least one shape (overall, or
    among those without direct loads), their occupancy, and each shape's
    times (0 beyond TABLE_CUT x its best).
    Configurations the built library no longer has are left out."""
    import dense_fp32_matrix_02_amd as sg

    known = set(sg.config_names())
    results = [dict(r, times_ms={n: t for n, t in r["times_ms"].items() if n in known}) for r in results]
    with open(path, "w") as f:
        # rows record the repetitions they were timed with; older ones take `reps`
        counts = sorted({r.get("reps", reps) for r in results}) or [reps]
        text = str(counts[0]) if len(counts) == 1 else f"{counts[0]} to {counts[-1]}"
        most = max((r.get("passes", 1) for r in results), default=1)
        passes = f", the least over up to {most} passes" if most > 1 else ""
        f.write(TABLE_HEADER.format(reps=text, passes=passes, cut=TABLE_CUT))
        blocks = []
        for ops in OPS_NAMES:
            sk_rows = [r for r in results if r.get("ops", "nn") == ops and r.get("streamk_ms")]
            rows = [r for r in results if r.get("ops", "nn") == ops and r.get("batch", 1) == 1
                    and not r.get("streamk_grid")]
            rows = [r for r in rows if any(n.startswith("mfma") for n in r["times_ms"])]
            if not rows:
                continue
            occ = {}
            for r in rows:
                occ.update(r.get("occupancy", {}))
            # the fastest configuration of each shape, then the fastest of those
            # without direct loads: direct-LDS configurations cannot serve
            # problems off their direct path (misaligned operands), so the
            # table also keeps the best register-staged one at every shape
            best = [min((n for n in r["times_ms"] if n.startswith("mfma")), key=r["times_ms"].get) for r in rows]
            staged = [min((n for n in r["times_ms"] if n.startswith("mfma") and "_lds" not in n),
                          key=r["times_ms"].get) for r in rows]
            cands = sorted(set(best), key=best.index)
            cands += [n for n in sorted(set(staged), key=staged.index) if n not in cands]
            missing = [n for n in cands if n not in occ]
            if missing:
                raise ValueError(f"no occupancy recorded for {missing} ({ops})")
            f.write(f"\n// op pair {ops}: {len(cands)} candidates, {len(rows)} shapes\n")
            f.write(f"static const TableConfig kCand_{ops}[] = {{\n")
            for n in cands:
                f.write(f'    {{"{n}", {occ[n]}}},\n')
            f.write("};\n")
            f.write(f"static const TableShape kShapes_{ops}[] = {{\n")
            for r in rows:
                f.write(f'    {{{r["M"]}, {r["N"]}, {r["K"]}}},\n')
            f.write("};\n")
            f.write(f"static const float kTimes_{ops}[] = {{\n")
            for r in rows:
                t = r["times_ms"]
                b = min(t[n] for n in t if n.startswith("mfma"))
                cells = []
                for n in cands:
                    v = t.get(n)
                    cells.append("0" if v is None or v > TABLE_CUT * b else f"{v * 1e3:.5g}")
                f.write("    " + ", ".join(cells) + ",\n")
            f.write("};\n")
            # every configuration's median time per unit of modelled busy time
            # over the shapes, for problems without a measured shape nearby
            names = sorted({n for r in rows for n in r["times_ms"] if n.startswith("mfma")})
            f.write(f"static const TableNorm kNorm_{ops}[] = {{\n")
            for n in names:
                if n not in occ:
                    raise ValueError(f"no occupancy recorded for {n} ({ops})")
                geo = config_geometry(n)
                ratios = [r["times_ms"][n] * 1e3 / busy_time(*geo, occ[n], r["M"], r["N"], r["K"])
                          for r in rows if n in r["times_ms"]]
                f.write(f'    {{"{n}", {occ[n]}, {statistics.median(ratios):.5g}}},\n')
            f.write("};\n")
            # stream-K: each configuration's time per slab of the evenly dealt
            # work, beyond the fixed overhead, median over the measured shapes
            sk = streamk_norms(sk_rows, occ)
            if sk:
                f.write(f"static const TableNorm kStreamK_{ops}[] = {{\n")
                for n, (o, us) in sk.items():
                    f.write(f'    {{"{n}", {o}, {us:.5g}}},\n')
                f.write("};\n")
            blocks.append((ops, len(cands), len(rows), len(names), len(sk)))
        split_rows = [r for r in results if r.get("splitk_ms") and r.get("batch", 1) == 1
                      and r.get("ops", "nn") == "nn"]
        f.write("\n// split-K: per measured shape {M, N, K, fastest split count} among 1, 2, 4, ..., 64\n")
        f.write("static const SplitShape kSplitShapes[] = {\n")
        for r in split_rows:
            t = {int(k): v for k, v in r["splitk_ms"].items()}
            f.write(f'    {{{r["M"]}, {r["N"]}, {r["K"]}, {min(t, key=t.get)}}},\n')
        f.write("    {0, 0, 0, 0},  // sentinel\n};\n")
        f.write("\nstatic const TableBlock kTableBlocks[] = {\n")
        for ops, nc, nr, nn, ns in blocks:
            f.write(f"    {{{int(ops[0] == 't')}, {int(ops[1] == 't')}, {nc}, {nr}, kCand_{ops}, kShapes_{ops}, "
                    f"kTimes_{ops}, {nn}, kNorm_{ops}, {ns}, {f'kStreamK_{ops}' if ns else 'nullptr'}}},\n")
        f.write("};\n")


if __name__ == "__main__":
    main()
