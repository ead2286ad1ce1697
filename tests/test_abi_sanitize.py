"""Host-only sanitizer run of the C ABI's argument checks (CPU).

tests/sanitize/abi_sanitize.cpp calls every entry point of include/lwg.h, a
fixed list of refusals and a seeded sweep of extreme arguments, against
lwg_abi.hip built with AddressSanitizer and UndefinedBehaviorSanitizer and the
stand-in launchers of tests/sanitize/abi_stubs.cpp, which check every launcher
precondition. No GPU and no kernel code are involved: the stand-ins launch
nothing, and the pointers passed are never dereferenced.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_checks_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = tmp_path / "abi_sanitize"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "layernorm_window_gather_amd", "csrc"), "-I", HERE,
           "-x", "c++", os.path.join(ROOT, "layernorm_window_gather_amd", "csrc", "lwg_abi.hip"), "-x", "none",
           os.path.join(HERE, "abi_stubs.cpp"), os.path.join(HERE, "abi_sanitize.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe), "200000"], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 launcher precondition violations, 0 failures" in run.stdout, run.stdout


def test_abi_checks_with_concurrent_callers_under_tsan(tmp_path):
    """tests/sanitize/abi_threads.cpp: 8 threads call the C ABI at once, each
    mixing refusals that carry its own value with accepted calls, and check
    that lwg_last_error() always reports the calling thread's own outcome. Built
    with ThreadSanitizer, which fails the run on any data race."""
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = tmp_path / "abi_threads"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-fno-omit-frame-pointer", "-pthread",
           "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "layernorm_window_gather_amd", "csrc"), "-I", HERE,
           "-x", "c++", os.path.join(ROOT, "layernorm_window_gather_amd", "csrc", "lwg_abi.hip"), "-x", "none",
           os.path.join(HERE, "abi_stubs.cpp"), os.path.join(HERE, "abi_threads.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    run = subprocess.run([str(exe), "8", "20000"], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr[-3000:]
    assert "0 launcher precondition violations, 0 failures" in run.stdout, run.stdout
    assert "WARNING: ThreadSanitizer" not in run.stderr, run.stderr[-3000:]


def test_multiply_shift_division_is_exact(tmp_path):
    """make_fastdiv (the reciprocals the window-table kernels divide by): exact
    for every divisor up to 2^16 and sampled divisors up to 2^31 - 1, at the
    dividends around the first and last multiples below 2^31 and at random
    points (tests/sanitize/fastdiv_check.cpp)."""
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = tmp_path / "fastdiv_check"
    cmd = [gxx, "-std=c++17", "-O2", "-fsanitize=undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "layernorm_window_gather_amd", "csrc"),
           os.path.join(HERE, "fastdiv_check.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert " 0 wrong" in run.stdout, run.stdout
