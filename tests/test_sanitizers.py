"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, CPU only:
the C oracle (gcc, -fsanitize=address,undefined) runs every oracle pin, and
the HIP library with its host code instrumented (hipcc -Xarch_host
-fsanitize=..., device code as usual) runs the argument-validation tests of
the C ABI.  Each runs in a child process with the sanitizer runtime
preloaded; the first report aborts it."""

import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _run_tests(env_extra, files):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *files], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and not any(s in out for s in REPORTS), out[-4000:]
    return out


def test_oracle_under_sanitizers():
    import oracle

    with tempfile.TemporaryDirectory() as d:
        lib = oracle.build(os.path.join(d, "liboracle_san.so"), sanitize=True)
        rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                            text=True).stdout.strip()
        ub = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True,
                            text=True).stdout.strip()
        files = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
        _run_tests({"ORACLE_LIB": lib, "LD_PRELOAD": f"{rt}:{ub}"}, files)


def test_abi_validation_under_sanitizers():
    from expert_token_routing_router_amd import build as hip_build

    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    with tempfile.TemporaryDirectory() as d:
        lib = hip_build.build(out=os.path.join(d, "libmoe_san.so"), sanitize=True)
        _run_tests({"MOE_MI355X_LIB": lib, "LD_PRELOAD": rt},
                   [os.path.join(ROOT, "tests", "test_abi.py")])
