"""Builds the oracle library in place with gcc (fp64, no fast-math, no FMA contraction)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose=False):
    out = os.path.join(HERE, "liboracle.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-Wall", "-o", out, os.path.join(HERE, "oracle.c"), "-lm"],
                   check=True)
    return [out]


if __name__ == "__main__":
    print(build(verbose=True))
