"""The C ABI from a native caller: tests/native/abi_caller (built by
__graft_entry__.build()) allocates with hipMalloc, calls the plain, general,
batched and split-K entry points on its own stream, checks each against the
CPU oracle bit for bit (integer inputs), and checks that argument errors come
back as codes. It runs as a child process, so no Python or torch state is
involved in its GPU work. A second child process loads the library before
torch and then runs on torch's stream."""
from __future__ import annotations

import os
import subprocess

import pytest

from tests import _gpu as G

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_caller")


def test_native_caller_passes():
    G.require_gpu()
    if not os.path.exists(EXE):
        pytest.fail("tests/native/abi_caller is missing: run __graft_entry__.build() first")
    print("[gpu] native C ABI caller", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, f"native caller failed (rc={r.returncode}):\n{r.stdout}\n{r.stderr}"
    assert "ALL PASSED" in r.stdout


LOAD_BEFORE_TORCH = r'''
import sys
sys.path.insert(0, sys.argv[1])
import dense_fp32_matrix_02_amd as sg
sg.load()                       # the library first, before any torch import of ours
n = sg.sgemm_mi355_num_configs()
import torch
a = torch.full((96, 80), 2.0, device="cuda")
b = torch.full((80, 72), 3.0, device="cuda")
c = sg.matmul(a, b)
torch.cuda.synchronize()
assert n > 0 and bool((c == 480.0).all()), c
print("LOAD-ORDER-OK")
'''


def test_library_loaded_before_torch_runs_on_torch_streams():
    """A process that loads the library before importing torch itself still
    launches on torch's streams: load() brings torch's HIP runtime in first,
    so the process holds one runtime. Run as a child process, whose first
    import is the package."""
    G.require_gpu()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("[gpu] library loaded before torch, child process", flush=True)
    r = subprocess.run(["python3", "-c", LOAD_BEFORE_TORCH, root], capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:])
    assert r.returncode == 0 and "LOAD-ORDER-OK" in r.stdout, r.stderr[-4000:]
