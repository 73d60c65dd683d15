"""The host planner and the C ABI's host paths under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

``plan.cpp`` and ``api.cpp`` are built with g++ (``-fsanitize=address,undefined``,
no recovery) into a host-only library in which every HIP runtime call and
kernel launcher is a stand-in that aborts (``tests/sanitize/hip_stubs.cpp``): a
plan without a device workspace and every argument check make no HIP call.
The CPU ABI tests (the 400 random geometries bit-exact against the plan spec,
the benchmark configurations, the error codes, the block-sparse page tables)
then run in a subprocess that loads the sanitizer library (``PKFA_LIB``) with
the ASan runtime preloaded. A canary with a planted out-of-bounds read, present
only in that library, shows that the instrumentation is live.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_fa_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _gxx():
    return shutil.which("g++")


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    if not _gxx() or not os.path.exists(os.path.join(ROCM, "include", "hip")):
        pytest.skip("g++ or the HIP headers are not available")
    out = str(tmp_path_factory.mktemp("asan") / "libpkfa_host_asan.so")
    cmd = [_gxx(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "sanitize", "hip_stubs.cpp"),
           "-o", out, "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _env(lib):
    runtime = subprocess.run([_gxx(), "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, PKFA_LIB=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONPATH=ROOT)
    return env


def test_sanitizer_is_live(asan_lib):
    code = ("import ctypes, os; lib = ctypes.CDLL(os.environ['PKFA_LIB']); "
            "lib.pkfa_sanitizer_canary(4)")
    r = subprocess.run([sys.executable, "-c", code], env=_env(asan_lib), capture_output=True,
                       text=True, timeout=120)
    # UBSan's object-size check or ASan's heap check stops the process first
    caught = "AddressSanitizer" in r.stderr or "runtime error" in r.stderr
    assert r.returncode != 0 and caught, r.stderr[-2000:]


def test_planner_and_abi_host_paths_clean_under_asan_ubsan(asan_lib):
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        "-q", "-p", "no:cacheprovider", "-k", "not probe"],
                       env=_env(asan_lib), capture_output=True, text=True, timeout=900, cwd=ROOT)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
