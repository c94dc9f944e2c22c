"""Build the native C ABI caller (tests/native/abi_caller) with hipcc.

Host code only: it includes include/sgemm_mi355.h, links the HIP library
(dense_fp32_matrix_02_amd/libsgemm_mi355.so) and the CPU oracle
(oracle/liboracle.so), and finds both at run time relative to its own
location, so the tree can move.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_caller.cpp")
EXE = os.path.join(HERE, "abi_caller")
PKG = os.path.join(ROOT, "dense_fp32_matrix_02_amd")
ORACLE = os.path.join(ROOT, "oracle")


def build() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = EXE + ".tmp"
    cmd = [hipcc, "-O2", "-std=c++17", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), SRC,
           "-L", PKG, "-lsgemm_mi355", "-L", ORACLE, "-loracle",
           "-Wl,-rpath,$ORIGIN/../../dense_fp32_matrix_02_amd", "-Wl,-rpath,$ORIGIN/../../oracle",
           "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(), file=sys.stderr)
