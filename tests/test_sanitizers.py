"""The oracle and the library's host code under AddressSanitizer + UBSan.

CPU only.  Each test builds the sanitized variant (the oracle with gcc, the
library's host pass with clang through hipcc; device code is unchanged) and
runs existing CPU tests against it in a child process that preloads the
matching sanitizer runtime.  A sanitizer report aborts the child, so the test
fails with the report in its message.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV_BASE = {
    "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
}


def _child(env_extra, args, timeout=600):
    env = dict(os.environ, **ENV_BASE, **env_extra)
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def _gcc_asan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                       text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return p


def _clang_asan():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    return hits[-1]


def test_oracle_tests_pass_under_asan_and_ubsan():
    import oracle
    oracle.build(force=True, sanitize=True)
    env = {"OASIS_ORACLE_SANITIZE": "1", "LD_PRELOAD": _gcc_asan()}
    rc, out = _child(env, ["-c", "import oracle; print(oracle.lib()._name)"])
    assert rc == 0 and "liboasis_oracle_san.so" in out, out[-3000:]
    rc, out = _child(env, ["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m",
                           "not gpu", "tests/test_oracle_pins.py",
                           "tests/test_oracle_trajectory.py"])
    assert rc == 0, out[-5000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-5000:]


def test_sanitized_oracle_reports_an_out_of_bounds_write():
    # The check above is only as good as the instrumentation: a top-K asked
    # for 6 ids into a 2-entry buffer must be reported.
    import oracle
    oracle.build(force=False, sanitize=True)
    env = {"OASIS_ORACLE_SANITIZE": "1", "LD_PRELOAD": _gcc_asan()}
    code = ("import ctypes, numpy as np, oracle\n"
            "L = oracle.lib()\n"
            "s = np.arange(8, dtype=np.float32); out = np.zeros(2, np.int32)\n"
            "L.orc_topk(s.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), 8, 6,\n"
            "           out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))\n")
    rc, out = _child(env, ["-c", code])
    assert rc != 0 and "heap-buffer-overflow" in out, out[-3000:]


def _sanitized_library():
    from lookahead_sparse_kv_oasis_amd import build as hipbuild
    if not os.path.exists(hipbuild.HIPCC):
        pytest.skip("hipcc is not installed")
    srcs = hipbuild.sources() + glob.glob(os.path.join(hipbuild.CSRC, "*.h")) + \
        glob.glob(os.path.join(ROOT, "include", "*.h"))
    lib = hipbuild.SAN_LIB
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(map(os.path.getmtime, srcs)):
        hipbuild.build(sanitize=True)
    return lib


def test_library_host_code_passes_the_abi_tests_under_asan_and_ubsan():
    lib = _sanitized_library()
    env = {"OASIS_LIBRARY": lib, "LD_PRELOAD": _clang_asan()}
    rc, out = _child(env, ["-c", "import lookahead_sparse_kv_oasis_amd as p; print(p.lib()._name)"])
    assert rc == 0 and "liboasis_san.so" in out, out[-3000:]
    rc, out = _child(env, ["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m",
                           "not gpu", "tests/test_library_abi.py"])
    assert rc == 0, out[-5000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-5000:]
