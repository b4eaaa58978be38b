"""Build the HIP verifier library in-tree for gfx950.

    python rejection_sampling_verification_amd/build.py

compiles csrc/sd_verify.hip (the verifier) and csrc/sd_ngram.hip (the n-gram
proposer) into libsdverify.so next to this file, then the test suite's
C-ABI caller tests/c_abi_check (plain C++ against include/sd_verify.h and the
library, no Python) and tests/gumbel_probe (the device Gumbel variates for
every possible uniform).
"""
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SOURCES = [os.path.join(PKG_DIR, "csrc", name) for name in ("sd_verify.hip", "sd_ngram.hip")]
LIBRARY = os.path.join(PKG_DIR, "libsdverify.so")
C_CHECK_SOURCE = os.path.join(ROOT, "tests", "c_abi_check.cpp")
C_CHECK = os.path.join(ROOT, "tests", "c_abi_check")
GUMBEL_PROBE_SOURCE = os.path.join(ROOT, "tests", "gumbel_probe.hip")
GUMBEL_PROBE = os.path.join(ROOT, "tests", "gumbel_probe")
ARCH = "gfx950"


def hipcc_path():
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def compile_command(output=LIBRARY, extra=()):
    return [
        hipcc_path(), "-O3", f"--offload-arch={ARCH}", "-std=c++17", "-shared", "-fPIC",
        # packed fp32 VALU forms are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # every atomic here is issued by one lane; the wave-combining rewrite
        # would wait for an atomic's return right after issuing it
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        "-I", os.path.join(ROOT, "include"),
        *extra, "-o", output, *SOURCES,
    ]


def c_check_command(output=C_CHECK):
    return [
        hipcc_path(), "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), C_CHECK_SOURCE,
        "-L", PKG_DIR, "-lsdverify", "-Wl,-rpath,$ORIGIN/../rejection_sampling_verification_amd",
        "-o", output,
    ]


def build_library(verbose=False):
    tmp = LIBRARY + ".tmp"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    os.replace(tmp, LIBRARY)
    if verbose:
        print("built", LIBRARY)
    if os.path.exists(C_CHECK_SOURCE):
        cmd = c_check_command(C_CHECK + ".tmp")
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
        os.replace(C_CHECK + ".tmp", C_CHECK)
        if verbose:
            print("built", C_CHECK)
    if os.path.exists(GUMBEL_PROBE_SOURCE):
        cmd = [hipcc_path(), "-O3", f"--offload-arch={ARCH}", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               GUMBEL_PROBE_SOURCE, "-o", GUMBEL_PROBE + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
        os.replace(GUMBEL_PROBE + ".tmp", GUMBEL_PROBE)
        if verbose:
            print("built", GUMBEL_PROBE)
    return LIBRARY


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
