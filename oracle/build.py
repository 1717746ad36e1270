"""Build the CPU oracle (plain C, gcc, OpenMP) into oracle/liboracle.so.

Test infrastructure: only the tests, the smoke check and the CPU-baseline leg
of the benchmark load the result."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = [os.path.join(HERE, "oracle.c"), os.path.join(HERE, "quant.c")]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", *SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
