"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so.

gcc, -O2, OpenMP, no fast-math and no FMA contraction, so that every fp32
division is the IEEE correctly rounded one and every double product is
rounded on its own.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "ptpc_oracle.c")
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", LIB + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
