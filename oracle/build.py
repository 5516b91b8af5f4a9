"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-Wall", "-Wextra", "-shared", "-fPIC", src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
