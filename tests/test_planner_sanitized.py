"""The planner and the host half of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer.

planner.cpp + abi_host.cpp + abi_host_only.cpp (no HIP) are compiled with
g++ -fsanitize=address,undefined into a host-only library, and the planner
test files run against it in a child process (BSA_LIBRARY names the library,
LD_PRELOAD puts the ASan runtime first).  Any heap overflow, use after free or
undefined behaviour in the planner aborts that run with the sanitizer report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_attention_bsr_amd", "csrc")
OUT_DIR = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT_DIR, "libbsa_host_asan.so")
SOURCES = ["planner.cpp", "abi_host.cpp", "abi_host_only.cpp"]
PLANNER_TESTS = ["tests/test_planner.py", "tests/test_planner_masks.py"]


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def asan_lib():
    if os.environ.get("BSA_LIBRARY"):
        pytest.skip("already running against another build")
    if _runtime("libasan.so") is None or _runtime("libubsan.so") is None:
        pytest.skip("g++ has no ASan/UBSan runtime here")
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fPIC", "-shared", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-3000:]
    return LIB


def test_planner_tests_pass_under_asan_and_ubsan(asan_lib):
    env = dict(os.environ)
    env.update({
        "BSA_LIBRARY": asan_lib,
        "LD_PRELOAD": _runtime("libasan.so"),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    proc = subprocess.run([sys.executable, "-m", "pytest", *PLANNER_TESTS, "-x", "-q", "-m", "not gpu",
                           "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=900)
    out = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert proc.returncode == 0, out[-6000:]
    assert " passed" in proc.stdout
