"""Build the CPU oracle shared library (oracle/liboracle.so) with g++.

Test infrastructure: the oracle is compiled with strict IEEE settings (no
contraction of a*b+c into an FMA, no fast-math) so each float operation in
ep_oracle.cpp is a single correctly rounded binary32 operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ep_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

CXXFLAGS = ["-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
            "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["g++", *CXXFLAGS, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
