"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer: the C-ABI's
argument checks, policy choice, split and stream-K sizing (a host-only build of every
translation unit of the library) and the oracle, exercised by the CPU tests in a child
process with the sanitizer runtime preloaded.  Any report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"


def _asan_runtime():
    try:
        out = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True, timeout=60).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        out = ""
    for cand in (out, ASAN_RT):
        if cand and os.path.isabs(cand) and os.path.exists(cand):
            return cand
    return None


def test_host_code_under_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime in this toolchain")
    sys.path.insert(0, ROOT)
    from dense_blas3_gemm_amd import build as b
    import oracle
    lib = b.build_sanitized()
    olib = oracle.build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        # the interpreter's own allocations are never freed at exit; leaks are not the question
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
        "DBGEMM_LIB": lib,
        "ORACLE_LIB": olib,
        "OMP_NUM_THREADS": "2",
    })
    tests = [os.path.join(ROOT, "tests", f) for f in ("test_abi.py", "test_oracle.py", "test_oracle_blas3.py",
                                                        "test_tolerance.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and " skipped" not in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
