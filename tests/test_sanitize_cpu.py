"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two builds, each loaded into a fresh Python process with the sanitizer
runtime preloaded:

  * the CPU oracle (``oracle/ref_sgemm.c``), compiled by gcc with
    -fsanitize=address,undefined, runs its four functions on padded,
    transposed, empty and K = 0 problems and must still give the exact
    closed-form results; a copy with a planted one-past-the-row read must be
    stopped by the sanitizer, which shows the check is live;
  * the host side of the library (``csrc/sgemm_api.hip``: argument
    validation with 128-bit extents, the selection and its table lookups,
    split-K and stream-K planning, the tile map), compiled by hipcc with the
    sanitizers on the host pass only and linked with the library's normal
    kernel objects, runs the validation and selection checks of
    ``tests/test_abi_cpu.py``. No kernel is launched.

A sanitizer report makes the child process exit with an error, so each test
asserts a clean exit and no report in its output.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=23",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    "OMP_NUM_THREADS": "2",
}


def _run(preload: str, script: str, timeout: int = 600):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env["LD_PRELOAD"] = preload
    env["PYTHONPATH"] = ROOT
    return subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True,
                          timeout=timeout, cwd=ROOT)


def _clean(r) -> bool:
    out = r.stdout + r.stderr
    return r.returncode == 0 and "AddressSanitizer" not in out and "runtime error" not in out


# ---------------------------------------------------------------- the oracle

ORACLE_SCRIPT = textwrap.dedent('''
    import numpy as np
    import oracle
    lib = oracle.load(LIB)
    rng = np.random.default_rng(5)

    def ints(r, c):
        return rng.integers(-4, 5, size=(r, c)).astype(np.float32)

    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (17, 9, 33), (64, 48, 129), (5, 70, 2)]:
        A, B = ints(M, K), ints(K, N)
        exact = A.astype(np.float64) @ B.astype(np.float64)
        # padded rows on every operand, C padding untouched
        Ap = np.full((M, K + 3), np.nan, np.float32); Ap[:, :K] = A
        Bp = np.full((K, N + 5), np.nan, np.float32); Bp[:, :N] = B
        Cp = np.full((M, N + 2), -7.0, np.float32)
        oracle.sgemm_f32(Ap[:, :K], Bp[:, :N], out=Cp[:, :N], lib=lib)
        assert np.array_equal(Cp[:, :N], exact) and np.all(Cp[:, N:] == -7.0)
        C64, S = oracle.sgemm_f64_abs(Ap[:, :K], Bp[:, :N], lib=lib)
        assert np.array_equal(C64, exact)
        assert np.array_equal(S, np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64))
        for opA in (0, 1):
            for opB in (0, 1):
                As = np.ascontiguousarray(A.T) if opA else A
                Bs = np.ascontiguousarray(B.T) if opB else B
                C0 = ints(M, N)
                C = C0.copy()
                oracle.sgemm_ex_f32(opA, opB, 2.0, As, Bs, -1.0, C, lib=lib)
                assert np.array_equal(C, 2.0 * exact - C0)
                P, S2 = oracle.sgemm_ex_f64_abs(opA, opB, As, Bs, lib=lib)
                assert np.array_equal(P, exact)
    # K = 0: C = 0; M = 0: nothing; alpha = 0: A and B not read
    C = np.full((4, 6), np.nan, np.float32)
    oracle.sgemm_f32(np.zeros((4, 0), np.float32), np.zeros((0, 6), np.float32), out=C, lib=lib)
    assert np.all(C == 0.0)
    oracle.sgemm_f32(np.zeros((0, 3), np.float32), np.ones((3, 6), np.float32),
                     out=np.zeros((0, 6), np.float32), lib=lib)
    C = np.ones((3, 4), np.float32)
    oracle.sgemm_ex_f32(0, 0, 0.0, np.zeros((0, 0), np.float32), np.zeros((0, 0), np.float32), 3.0, C,
                        K=5, lib=lib)
    assert np.all(C == 3.0)
    print("ORACLE-SANITIZED-OK")
''')


def _gcc_sanitized_oracle(tmp_path, source: str) -> str:
    from oracle import build as obuild

    src = tmp_path / "ref_sgemm_san.c"
    src.write_text(source)
    out = str(tmp_path / "liboracle_san.so")
    obuild.compile_oracle(str(src), out, extra=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                                "-fno-omit-frame-pointer", "-g", "-Wno-error"))
    return out


def _gcc_asan_runtime() -> str:
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


@pytest.fixture(scope="module")
def gcc_ok():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return _gcc_asan_runtime()


def test_oracle_is_clean_under_asan_and_ubsan(gcc_ok, tmp_path):
    from oracle import build as obuild

    lib = _gcc_sanitized_oracle(tmp_path, open(obuild.SRC).read())
    r = _run(gcc_ok, ORACLE_SCRIPT.replace("LIB)", repr(lib) + ")"))
    assert _clean(r), r.stdout[-3000:] + r.stderr[-6000:]
    assert "ORACLE-SANITIZED-OK" in r.stdout


def test_planted_out_of_bounds_read_is_reported(gcc_ok, tmp_path):
    """The same run on a copy of the oracle whose inner loop reads one value
    past the end of each row of B must be stopped by AddressSanitizer: the
    last row of B ends at the end of its numpy buffer."""
    from oracle import build as obuild

    src = open(obuild.SRC).read()
    old = "float p = aik * b[j];"
    assert old in src
    lib = _gcc_sanitized_oracle(tmp_path, src.replace(old, "float p = aik * b[j + 1];", 1))
    script = textwrap.dedent(f'''
        import numpy as np
        import oracle
        lib = oracle.load({lib!r})
        A = np.ones((3, 4), np.float32)
        B = np.ones((4, 5), np.float32)   # unpadded: its last row ends at the end of the buffer
        oracle.sgemm_f32(A, B, lib=lib)
        print("NOT-CAUGHT")
    ''')
    r = _run(gcc_ok, script)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr and "NOT-CAUGHT" not in r.stdout, \
        r.stdout[-2000:] + r.stderr[-4000:]


# ---------------------------------------------------------------- host dispatch

def _clang_asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    return hits[-1]


def _sanitized_host_library(tmp_path) -> str:
    """sgemm_api.hip with ASan and UBSan on the host pass (the device pass is
    untouched), linked with the normal kernel objects into a library of its
    own."""
    from dense_fp32_matrix_02_amd import build as b

    objs = []
    for src in b.SOURCES:
        if src == "sgemm_api.hip":
            continue
        obj = os.path.join(b.OBJDIR, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(obj):
            b._compile(src)
        objs.append(obj)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-shared-libasan"]
    api_obj = str(tmp_path / "sgemm_api_san.o")
    cmd = [b.hipcc(), *b.HIPFLAGS, "-g", *san, "-c", os.path.join(b.CSRC, "sgemm_api.hip"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    lib = str(tmp_path / "libsgemm_mi355_san.so")
    # no sanitizer flag at the link: the instrumented object's __asan_* and
    # __ubsan_handle_* references resolve at load time against the preloaded
    # runtime, which carries both
    cmd = [b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", api_obj, *objs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "the host code is not instrumented"
    return lib


HOST_SCRIPT = textwrap.dedent('''
    import ctypes, itertools, random
    from dense_fp32_matrix_02_amd import _binding
    _binding.load(LIB)
    import dense_fp32_matrix_02_amd as sg
    assert hasattr(ctypes.CDLL(None), "__asan_init"), "the sanitizer runtime is not loaded"
    import tests.test_abi_cpu as t
    for args, code in t.VALIDATION_CASES:
        t.test_validation_codes(args, code)
    for fn in ("sgemm_mi355", "sgemm_mi355_valu"):
        t.test_entry_points_reject_before_any_hip_call(fn)
    for name in ("test_with_config_rejects_unknown_ids", "test_config_metadata",
                 "test_validate_ex_ops_and_leading_dims", "test_validate_ex_batch_and_strides",
                 "test_validate_ex_alpha_zero_and_k_zero_skip_a_and_b",
                 "test_general_entry_points_reject_before_any_hip_call", "test_config_ops_and_config_op_mismatch",
                 "test_config_staging_follows_the_direct_load_rules"):
        getattr(t, name)()
    for tm, tn, g in [(1, 1, 4), (3, 5, 2), (24, 16, 4), (13, 29, 8), (64, 3, 16)]:
        t.test_tile_map_is_a_bijection(tm, tn, g)
    # the selection and the split-K / stream-K planning over many shapes,
    # extremes included
    rnd = random.Random(7)
    sides = [0, 1, 2, 3, 31, 64, 255, 1000, 3001, 8192, 65535, 2 ** 20, 2 ** 31 - 1025]
    shapes = list(itertools.product(sides[:9], repeat=3)) + [
        tuple(rnd.choice(sides) for _ in range(3)) for _ in range(300)]
    A0, B0 = 0x10000000, 0x20000000
    for (M, N, K) in shapes:
        for opA in (0, 1):
            for opB in (0, 1):
                for batch in (1, 7, 70000):
                    c = sg.sgemm_mi355_select_config_ex(opA, opB, M, N, K, batch)
                    assert 0 <= c < sg.sgemm_mi355_num_configs()
                s, c = sg.sgemm_mi355_select_splitk(opA, opB, M, N, K)
                assert s >= 1 and 0 <= c < sg.sgemm_mi355_num_configs()
                assert sg.sgemm_mi355_select_streamk(opA, opB, M, N, K) >= -1
        sg.sgemm_mi355_splitk_workspace_size(M, N, K, 16)
        sg.sgemm_mi355_selected_config(M, N, K, A0, max(K, 1), B0, max(N, 1))
        sg.sgemm_mi355_selected_config(M, N, K, A0 + 4, max(K, 1) + 1, B0, max(N, 1))
        sg.sgemm_mi355_validate(M, N, K, A0, max(K, 1), B0, max(N, 1), 0x30000000, max(N, 1))
    print("HOST-SANITIZED-OK")
''')


def test_host_dispatch_is_clean_under_asan_and_ubsan(tmp_path):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    runtime = _clang_asan_runtime()
    lib = _sanitized_host_library(tmp_path)
    r = _run(runtime, HOST_SCRIPT.replace("LIB)", repr(lib) + ")"))
    assert _clean(r), r.stdout[-3000:] + r.stderr[-6000:]
    assert "HOST-SANITIZED-OK" in r.stdout
