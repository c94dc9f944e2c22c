"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Flags: -O2 (plain IEEE single/double arithmetic, no fast-math), -ffp-contract=off
(no fused multiply-add, so each term is a rounded product then a rounded add),
-fopenmp (rows split over threads; results do not depend on the thread count).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ref_sgemm.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Werror"]


def compile_oracle(src: str = SRC, out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    return compile_oracle()


if __name__ == "__main__":
    print(build(), file=sys.stderr)
