"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the ABI's host side (abi.cpp: argument checks, workspace carving,
routing-output copies, the layer stack with steering, the static scratch,
the timing record) linked with host-only stand-ins of the kernels, and the
oracle, each driven through every entry point by a small program.  Any
sanitizer report or unexpected status fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
         "-fno-sanitize-recover=undefined"]


def _run(cmd, exe, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = p.stdout + p.stderr
    assert p.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert p.stdout.strip().startswith("ok"), out[-4000:]


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the HIP headers")
def test_abi_host_code_sanitized(tmp_path):
    exe = str(tmp_path / "drive_abi")
    cmd = ["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "bit_quantized_moe_q2_amd", "csrc", "abi.cpp"),
           os.path.join(SAN, "stub_device.cpp"), os.path.join(SAN, "drive_abi.cpp"), "-o", exe]
    _run(cmd, exe, tmp_path)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_sanitized(tmp_path):
    exe = str(tmp_path / "drive_oracle")
    cmd = ["gcc", "-std=c11", *FLAGS, "-fopenmp", "-ffp-contract=off",
           os.path.join(SAN, "drive_oracle.c"), os.path.join(ROOT, "oracle", "ds4q_oracle.c"),
           "-o", exe, "-lm"]
    _run(cmd, exe, tmp_path)
