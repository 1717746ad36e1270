"""Build libbitmoe.so for gfx950 in-tree (hipcc, no JIT), and beside it
libbitmoe_checked.so, the same library built with BITMOE_CHECK_IDS = 1 (the
FFN and bucketing calls count the caller's routing ids outside [0, E) into
their workspace and read every id clamped into range).

    python -m bit_moe_amd.build      # or bit_moe_amd.build.build()
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libbitmoe.so")
LIB_CHECKED = os.path.join(HERE, "libbitmoe_checked.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.cpp", "plan.cpp", "cache.cpp", "dequant.hip", "route.hip", "bucket.hip", "decode.hip", "prefill.hip", "noalloc.hip", "quant.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(job) -> str:
    src, checked = job
    obj = os.path.join(OBJ, ("checked_" if checked else "") + os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DBITMOE_CHECK_IDS=1"] if checked else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg:
        print(msg)
    return obj


def build(jobs: int = 6) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, [(src, c) for c in (False, True) for src in SOURCES]))
    for lib, part in ((LIB, objs[:len(SOURCES)]), (LIB_CHECKED, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *part], check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build())
