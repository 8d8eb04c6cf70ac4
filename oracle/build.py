"""Build the fp64 CPU oracle (plain C, gcc) into oracle/libmsda_oracle.so.

Test infrastructure only: the product library never links this.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "msda_oracle.c")
LIB = os.path.join(HERE, "libmsda_oracle.so")


def build(verbose: bool = False) -> str:
    # No fast-math and no FMA contraction: every operation rounds as written.
    # OpenMP only splits whole queries / (image, head) pairs over threads
    # (serial unless msda_oracle_set_threads asks for more).
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fopenmp",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
