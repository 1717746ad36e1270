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
    rc, out = _run(_host_build(exe, "abi_main.cpp"))
    assert rc == 0, out
    rc, out = _run([exe], ENV)
    assert rc == 0 and "ok" in out, out
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out


def _host_build(exe, driver):
    """g++ line for the library's host code (validation, planning, the expert
    cache) with launcher stand-ins and the HIP runtime stand-in, under ASan
    and UBSan: no GPU and no HIP runtime involved."""
    csrc = os.path.join(ROOT, "bit_moe_amd", "csrc")
    san = os.path.join(ROOT, "tests", "sanitize")
    return ["g++", "-std=c++17", *SAN, "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-o", exe,
            os.path.join(csrc, "api.cpp"), os.path.join(csrc, "plan.cpp"), os.path.join(csrc, "cache.cpp"),
            os.path.join(san, "stub_launch.cpp"), os.path.join(san, "hip_standin.cpp"), os.path.join(san, driver)]


def _lru_model(steps, E, slots):
    """Reference residency policy: distinct experts in first-appearance
    order keep their slot; a missing one takes the lowest empty slot, else
    the least recently used slot not used in this step (lowest on ties)."""
    slot_of, expert_in, last = {}, [-1] * slots, [-1] * slots
    hits = misses = 0
    out = []
    for t, ids in enumerate(steps, start=1):
        distinct = list(dict.fromkeys(ids))
        for e in distinct:
            if e in slot_of:
                last[slot_of[e]] = t
        loaded = 0
        for e in distinct:
            if e in slot_of:
                hits += 1
                continue
            empty = [j for j in range(slots) if expert_in[j] < 0]
            if empty:
                v = empty[0]
            else:
                v = min((j for j in range(slots) if last[j] < t), key=lambda j: (last[j], j))
                del slot_of[expert_in[v]]
            expert_in[v], slot_of[e], last[v] = e, v, t
            misses += 1
            loaded += 1
        out.append(([slot_of[e] for e in ids], loaded, list(expert_in), hits, misses))
    return out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP runtime headers not available")
def test_expert_cache_policy_and_copies_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "cache_san")
    rc, out = _run(_host_build(exe, "cache_main.cpp"))
    assert rc == 0, out
    rc, out = _run([exe], ENV)
    assert rc == 0 and "cache sanitizer driver: ok" in out, out
    steps = [[3, 5], [5, 1, 3, 6], [0, 7], [7, 0, 3, 3], [2, 4, 6, 1], [1, 1], [5, 6, 7, 0], [2, 2, 2, 2], [4, 3]]
    got = []
    for line in out.splitlines():
        if not line.startswith("step"):
            continue
        a, b, c, d = line[4:].split("|")
        hits, misses = int(d.split()[1]), int(d.split()[3])
        got.append(([int(v) for v in a.split()], int(b.split()[1]), [int(v) for v in c.split()[1:]], hits, misses))
    assert got == _lru_model(steps, 8, 4)
