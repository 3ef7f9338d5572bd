"""The C-ABI host layer (argument checks, split planning, workspace sizing,
plan description, dispatch) built on the host alone with AddressSanitizer and
UndefinedBehaviorSanitizer, the kernel launchers replaced by stand-ins that
check and record what they are handed (tests/host_sanitize/).  The driver
sweeps valid shapes (the plan must agree with the launch, the workspace size
must be exact) and a list of invalid arguments (each refused, nothing
launched).  Any out-of-bounds access, signed overflow or bad shift aborts it.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "paged_kv_cache_195_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_host_layer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "pa_host_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", HERE, "-I", ROCM_INCLUDE,
           os.path.join(CSRC, "pa_api.cpp"), os.path.join(HERE, "stub_launchers.cpp"),
           os.path.join(HERE, "driver.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "host checks passed" in run.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_fast_div_matches_division(tmp_path):
    """The multiply-high division by the group size (csrc/fast_div.h) against
    plain division, built with UBSan: divisors 1..4096 and random larger
    ones, dividends around their multiples, near 2^31 and spread below it."""
    exe = str(tmp_path / "fast_div_check")
    cmd = ["g++", "-std=c++17", "-O1", "-fsanitize=undefined", "-fno-sanitize-recover=all",
           "-I", CSRC, os.path.join(HERE, "fast_div_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "fast_div checks passed" in run.stdout
