"""The C ABI's host code under AddressSanitizer, on the CPU: tests/c_abi_host_check.cpp
linked with the library's sources, AddressSanitizer on the host code only (the
kernels are built as usual and never launched).  It exercises every entry
point's argument checks, the workspace layout over the supported shapes, the
rates helper and the status strings."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rejection_sampling_verification_amd", "csrc")


@pytest.mark.timeout(900)
def test_host_code_under_address_sanitizer(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "c_abi_host_check")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_host_check.cpp"),
           os.path.join(CSRC, "sd_verify.hip"), os.path.join(CSRC, "sd_ngram.hip"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "host checks ok" in run.stdout
