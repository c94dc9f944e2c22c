"""Reader of the compiled-in tile table (dense_fp32_matrix_02_amd/csrc/
tile_table.inc) for the tests: per op pair, the candidate configurations
with their recorded occupancy, the measured shapes and the times."""
from __future__ import annotations

import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TABLE_PATH = os.path.join(ROOT, "dense_fp32_matrix_02_amd", "csrc", "tile_table.inc")
OP_PAIRS = {"nn": (0, 0), "nt": (0, 1), "tn": (1, 0), "tt": (1, 1)}


def read_table(path: str = TABLE_PATH):
    """{(opA, opB): (candidates [(name, occupancy)], shapes [(M, N, K)],
    times [[microseconds per candidate, as FP32]] per shape)}."""
    text = open(path).read()
    blocks = {}
    for ops, pair in OP_PAIRS.items():
        m = re.search(r"kCand_%s\[\] = \{(.*?)\n\};" % ops, text, re.S)
        if not m:
            continue
        cands = [(n, int(o)) for n, o in re.findall(r'\{"([^"]+)", (\d+)\}', m.group(1))]
        body = re.search(r"kShapes_%s\[\] = \{(.*?)\n\};" % ops, text, re.S).group(1)
        shapes = [tuple(int(x) for x in t) for t in re.findall(r"\{(\d+), (\d+), (\d+)\}", body)]
        body = re.search(r"kTimes_%s\[\] = \{(.*?)\n\};" % ops, text, re.S).group(1)
        cells = [float(np.float32(c.strip().rstrip("f"))) for c in body.split(",") if c.strip()]
        if len(cells) != len(shapes) * len(cands):
            raise ValueError(f"{ops}: {len(cells)} times for {len(shapes)} shapes x {len(cands)} candidates")
        times = [cells[i * len(cands):(i + 1) * len(cands)] for i in range(len(shapes))]
        blocks[pair] = (cands, shapes, times)
    return blocks


def read_split_table(path: str = TABLE_PATH):
    """The split-K block: [(M, N, K, fastest split count)] in table order."""
    text = open(path).read()
    body = re.search(r"kSplitShapes\[\] = \{(.*?)\n\};", text, re.S).group(1)
    rows = [tuple(int(x) for x in t) for t in re.findall(r"\{(\d+), (\d+), (\d+), (\d+)\}", body)]
    return [r for r in rows if r[0] > 0]  # without the sentinel


def nearest(shapes, M, N, K):
    """Index of the shape (first three fields M, N, K) nearest (M, N, K) in
    summed |log2| distance among those within a factor of two in every
    dimension (the first on a tie), or None."""
    import math
    near = None
    for i, e in enumerate(shapes):
        m, n, k = e[0], e[1], e[2]
        if M > 2 * m or m > 2 * M or N > 2 * n or n > 2 * N or K > 2 * k or k > 2 * K:
            continue
        d = abs(math.log2(M / m)) + abs(math.log2(N / n)) + abs(math.log2(K / k))
        if near is None or d < near[0]:
            near = (d, i)
    return None if near is None else near[1]


def read_norms(path: str = TABLE_PATH):
    """{(opA, opB): [(name, occupancy, median microseconds per busy unit)]}."""
    text = open(path).read()
    out = {}
    for ops, pair in OP_PAIRS.items():
        m = re.search(r"kNorm_%s\[\] = \{(.*?)\n\};" % ops, text, re.S)
        if m:
            out[pair] = [(n, int(o), float(np.float32(v)))
                         for n, o, v in re.findall(r'\{"([^"]+)", (\d+), ([0-9.eE+-]+)\}', m.group(1))]
    return out


def read_streamk(path: str = TABLE_PATH):
    """{(opA, opB): [(name, occupancy, microseconds per slab)]}: the stream-K block."""
    text = open(path).read()
    out = {}
    for ops, pair in OP_PAIRS.items():
        m = re.search(r"kStreamK_%s\[\] = \{(.*?)\n\};" % ops, text, re.S)
        if m:
            out[pair] = [(n, int(o), float(np.float32(v)))
                         for n, o, v in re.findall(r'\{"([^"]+)", (\d+), ([0-9.eE+-]+)\}', m.group(1))]
    return out
