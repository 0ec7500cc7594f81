"""The C ABI's validation and planning under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

tests/host/plan_fuzz.cpp links the library's host code (gemm_f16_api.cpp)
with stubs in place of the HIP runtime and the kernel launchers and drives
every entry point with a few hundred thousand argument sets: tile-edge,
large, out-of-range and negative dimensions, misaligned pointers, every
configuration index and split count.  Any out-of-bounds access, undefined
behaviour, launch of an invalid call or plan/launch mismatch fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="no clang++ with sanitizers")
def test_planning_and_validation_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_fuzz"
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "tiled_dense_gemm_fp16_amd", "csrc"),
           "-x", "c++", os.path.join(ROOT, "tiled_dense_gemm_fp16_amd", "csrc", "gemm_f16_api.cpp"),
           os.path.join(ROOT, "tests", "host", "plan_fuzz.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "0 failed checks" in run.stdout
