"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds two drivers with gcc/g++ (host code only, no device code):
 - the CPU oracle (oracle/oracle.c) run on a small seeded layer through
   every entry point (tests/sanitize/oracle_main.c);
 - the C ABI's validation, launch planning and workspace carving
   (bit_moe_amd/csrc/api.cpp, plan.cpp) over a sweep of shapes and token
   counts, with launcher stand-ins that queue nothing
   (tests/sanitize/abi_main.cpp, stub_launch.cpp).
Any sanitizer report aborts the driver (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=300)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    rc, out = _run(["gcc", "-std=c11", *SAN, "-Wall", "-o", exe, os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_main.c"), "-lm"])
    assert rc == 0, out
    rc, out = _run([exe], ENV)
    assert rc == 0 and "ok" in out, out
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP runtime headers not available")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    csrc = os.path.join(ROOT, "bit_moe_amd", "csrc")
    rc, out = _run(["g++", "-std=c++17", *SAN, "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-o", exe, os.path.join(csrc, "api.cpp"), os.path.join(csrc, "plan.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "stub_launch.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_main.cpp"),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    assert rc == 0, out
    # the HIP runtime (queried for the compute-unit count) keeps allocations
    # for the life of the process: leaks are not checked in this driver
    rc, out = _run([exe], dict(ENV, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1"))
    assert rc == 0 and "ok" in out, out
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out
