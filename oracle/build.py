"""Build the CPU oracle (oracle/libns_oracle.so) with gcc.

Test infrastructure: the GPU library never links or calls this library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ns_oracle.c")
LIB = os.path.join(HERE, "libns_oracle.so")

# -ffp-contract=off: every a*b+c is a rounded product then a rounded sum, as
# the formulas are written; no fused multiply-add changes the oracle's values.
CFLAGS = ["-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
          "-ffp-contract=off", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
