"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

abi.cpp holds only host code (argument checks, error strings, the device
check and the launches), so it is built here with g++ and
-fsanitize=address,undefined into a library of its own, linked with
host-only stand-ins for the kernel launchers (tests/sanitize/launch_stubs.cpp).
The argument-check tests of tests/test_abi_cpu.py then run against that
library in a child process with the sanitizer runtimes preloaded, any report
being fatal.  No GPU is used: on a machine with one the calls that pass every
check would reach the stand-ins, so the test runs only where there is none.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize", "libw4a8moe_sanitize.so")


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def sanitized_lib():
    if shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("needs g++ and the HIP headers")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("the sanitizer runtimes are not installed")
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present: calls that pass every check would reach the launcher stand-ins")
    except ImportError:
        pass
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{ROOT}/include", f"-I{ROOT}/quantized_grouped_gemm_token_amd/csrc",
           f"{ROOT}/quantized_grouped_gemm_token_amd/csrc/abi.cpp", f"{ROOT}/tests/sanitize/launch_stubs.cpp",
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(p for p in (asan, ubsan, env.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["W4A8_MOE_LIB"] = OUT
    return env


def test_sanitizer_runtime_is_active(sanitized_lib):
    code = ("import ctypes, os; L = ctypes.CDLL(os.environ['W4A8_MOE_LIB']); "
            "maps = open('/proc/self/maps').read(); print('libasan' in maps, 'libubsan' in maps)")
    r = subprocess.run([sys.executable, "-c", code], env=sanitized_lib, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["True", "True"]
    out = subprocess.run(["nm", "-D", OUT], capture_output=True, text=True).stdout
    assert "__asan_" in out and "__ubsan_" in out          # the library itself is instrumented


def test_abi_checks_under_sanitizers(sanitized_lib):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=sanitized_lib, capture_output=True, text=True, cwd=ROOT, timeout=300)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
