"""Host code built with g++ under AddressSanitizer and UBSan and driven
through seeded random and edge cases (CPU only; no device code is built):
the virtual-rank planners (fva_rlb_plan, fva_sasa_budget), and the C-ABI
argument validation (fva_api.hip) with its kernel launchers and HIP runtime
calls replaced by recording stubs."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "adaptive_block_sparse_reorder_amd", "csrc")


def test_host_planners_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    # the internal header uses the unqualified min/max that hipcc provides
    prelude = tmp_path / "prelude.h"
    prelude.write_text("#include <algorithm>\nusing std::max;\nusing std::min;\n")
    exe = tmp_path / "planners"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-include", str(prelude), "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "rlb_host.cpp"), os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-1000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    assert "all cases passed" in r.stdout


def test_api_validation_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    prelude = tmp_path / "prelude.h"
    prelude.write_text("#include <algorithm>\nusing std::max;\nusing std::min;\n")
    exe = tmp_path / "api_validation"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-include", str(prelude), "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-x", "c++", os.path.join(CSRC, "fva_api.hip"), "-x", "none",
           os.path.join(ROOT, "tests", "host_sanitize_api_driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-1000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    assert "all cases passed" in r.stdout
