"""The C ABI layer (fa_api.cpp: validation, planning, status strings) built
for the host with AddressSanitizer and UndefinedBehaviorSanitizer and driven
through every entry point by tests/abi_sanitize_driver.cpp, with the kernel
launchers replaced by recording stubs (no GPU, no HIP runtime).  Any
out-of-bounds access, use of freed memory, signed overflow, misaligned
access or other undefined behaviour on those paths aborts the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_52_amd", "csrc")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="g++ or the ROCm headers are missing")
def test_abi_layer_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_sanitize"
    # Host compiler only: no device code is built here.
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", ROCM_INCLUDE,
           os.path.join(CSRC, "fa_api.cpp"), os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # verify_asan_link_order=0: the environment may preload other libraries.
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all checks passed" in r.stdout
