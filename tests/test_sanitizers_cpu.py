"""Host AddressSanitizer + UndefinedBehaviorSanitizer builds (CPU only): the
oracle (every routine on small ragged inputs, several threads) and the C-ABI
validation of api.cpp (every entry point's argument checks and size
arithmetic over extreme shapes, with the kernel launchers stubbed).  Any
out-of-bounds access, leak, signed overflow or other undefined operation
aborts the driver, which fails the test."""
from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ROCM = "/opt/rocm"


def _run(exe: str):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, \
        (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.check_call(["gcc", "-std=c11", *SAN, "-o", exe, os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                           "-lm", "-lpthread"])
    assert "ok" in _run(exe)


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")), reason="no HIP runtime")
def test_abi_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "api_san")
    csrc = os.path.join(ROOT, "attention_output_projection_amd", "csrc")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
                           "-I", os.path.join(ROOT, "include"), "-I", csrc, "-o", exe,
                           os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"), os.path.join(csrc, "api.cpp"),
                           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")],
                          stderr=subprocess.DEVNULL)
    assert "ok" in _run(exe)
