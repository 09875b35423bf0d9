"""Build the CPU oracle shared library (test infrastructure only).

    python oracle/build.py

Compiles nvfp4_oracle.cpp with g++ -O2 -std=c++17 -ffp-contract=off (no fast-math), so that no
multiply-add is fused behind the code's back and every float operation is one IEEE binary32
operation, into oracle/libnvfp4_oracle.so.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.cpp")
LIB = os.path.join(HERE, "libnvfp4_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-pthread", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
