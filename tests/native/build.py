"""Build the native test programs with hipcc.

tests/native/abi_caller: host code only; it includes include/sgemm_mi355.h,
links the HIP library (dense_fp32_matrix_02_amd/libsgemm_mi355.so) and the
CPU oracle (oracle/liboracle.so), and finds both at run time relative to its
own location, so the tree can move.

tests/native/lds_probe: a stand-alone gfx950 program whose kernels repeat the
LDS access patterns of the GEMM kernels, for counter runs (rocprofv3 --pmc).
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
PROBE_SRC = os.path.join(HERE, "lds_probe.hip")
PROBE = os.path.join(HERE, "lds_probe")
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
    build_probe()
    return EXE


def build_probe() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = PROBE + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Wall", "-Werror",
           "-Wno-unused-command-line-argument", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for lds_probe.hip:\n{msg}")
    os.replace(tmp, PROBE)
    return PROBE


if __name__ == "__main__":
    print(build(), file=sys.stderr)
