"""The C ABI from a native caller: tests/native/abi_caller (built by
__graft_entry__.build()) allocates with hipMalloc, calls the plain, general,
batched and split-K entry points on its own stream, checks each against the
CPU oracle bit for bit (integer inputs), and checks that argument errors come
back as codes. It runs as a child process, so no Python or torch state is
involved in its GPU work."""
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
