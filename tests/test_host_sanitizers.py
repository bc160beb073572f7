"""The host half of the library (kk_host.cpp: table checks, work planning,
argument validation) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, with the host ABI tests run against that build.

The build links kk_host.cpp with stand-ins for the kernel launches
(tests/host_sanitize/launch_stubs.cpp, which abort if reached: no host ABI
test enqueues work).  The test runner is a child process with the ASan
runtime preloaded (the interpreter itself is not instrumented, so leak
checking is off); any sanitizer report fails it."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_decode_attention_kk_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _asan_runtime(gxx):
    p = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_host_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("needs g++ and the ROCm headers")
    asan = _asan_runtime(gxx)
    if asan is None:
        pytest.skip("g++ has no AddressSanitizer runtime")
    lib = str(tmp_path / "libkk_host_sanitized.so")
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fPIC", "-shared",
             os.path.join(CSRC, "kk_host.cpp"), os.path.join(ROOT, "tests", "host_sanitize", "launch_stubs.cpp"),
             "-o", lib, "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
             "-Wl,--no-undefined"]
    r = subprocess.run(build, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=asan, KK_HOST_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi_host.py")]
    r = subprocess.run(run, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, log
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, log
    assert "passed" in r.stdout and "sanitized build" in r.stdout, log
