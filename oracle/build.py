"""Build the CPU fp64 oracle (plain C, gcc, OpenMP) into oracle/liboracle.so.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg load the result; the product path never does.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lora_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# -ffp-contract=off keeps every a*b+c as a rounded product then a rounded sum,
# exactly as the source reads; no -ffast-math, so no reassociation either.
CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
