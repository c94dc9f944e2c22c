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
