"""Build the input generator's shared library (synth/libsynth.so).

    python synth/build.py

gen.c holds Philox4x32-10, Box-Muller and Fisher-Yates for the synthetic inputs; it is compiled with
gcc -O2 and no fast-math (log, sin, cos and sqrt are the C library's).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gen.c")
LIB = os.path.join(HERE, "libsynth.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall",
           "-Wextra", "-pthread", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
