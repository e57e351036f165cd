"""Host-side sanitizer runs: AddressSanitizer and UndefinedBehaviorSanitizer
over the oracle (its pins and the tolerance check's) and over the C-ABI's
host code (size queries, argument checks and error paths: the tests that need
no GPU).  Each runs in a child process with its compiler's ASan runtime
preloaded (gcc's for the oracle, clang's for the hipcc-built library, whose
device code is built as usual) and fails on any sanitizer report."""
import os
import subprocess
import sys

import pytest

import oracle
from submanifold_sparse_convolution_spconv_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: UndefinedBehavior")


def runtime(cmd):
    path = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"no sanitizer runtime from {' '.join(cmd)}")
    return path


def run_sanitized(preload, env_extra, tests):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for rep in REPORTS:
        assert rep not in out, out[-4000:]
    return out


def loaded_in_child(preload, env_extra, code, lib):
    """The sanitized build is the one a child process with this environment maps."""
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0", **env_extra)
    r = subprocess.run([sys.executable, "-c", code + "; print(open('/proc/self/maps').read())"], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert os.path.realpath(lib) in r.stdout


def test_oracle_under_asan_ubsan():
    lib = oracle.build(force=True, sanitize=True)
    pre, env = runtime(["gcc", "-print-file-name=libasan.so"]), {"SPCONV_ORACLE_LIB": lib}
    loaded_in_child(pre, env, "import oracle; oracle._load()", lib)
    out = run_sanitized(pre, env, ["tests/test_oracle.py", "tests/test_compare.py"])
    assert " passed" in out


@pytest.mark.timeout(900)
def test_capi_host_under_asan_ubsan():
    clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
    if not os.path.exists(clang):
        pytest.skip("no ROCm clang")
    lib = libbuild.build(sanitize=True)
    pre, env = runtime([clang, "-print-file-name=libclang_rt.asan-x86_64.so"]), {"SPCONV_LIB": lib}
    loaded_in_child(pre, env, "import submanifold_sparse_convolution_spconv_amd as sp; sp.load_library()", lib)
    out = run_sanitized(pre, env, ["tests/test_abi.py"])
    assert " passed" in out
