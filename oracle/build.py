"""Build the CPU oracle (oracle/liboracle.so) with the host C compiler.

Test infrastructure: the oracle is compiled without fast-math and without FMA
contraction so that every float expression is one IEEE binary32 operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        os.environ.get("CC", "gcc"), "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", "-Werror",
        "-Wno-unknown-pragmas",
        os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
